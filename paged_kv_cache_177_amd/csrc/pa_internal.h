// Internal interface between the C-ABI layer (pa_api.cpp) and the gfx950 kernels (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kBlock = 16;  // tokens per K/V block
constexpr int kMaxGridYZ = 65535;  // largest grid extent in y and z (rows, splits and heads go there)

// ---- split rule ------------------------------------------------------------------------------
// A row of n keys is cut into ceil(n / chunk) chunks of `chunk` tokens (the last one shorter);
// chunk depends only on head_dim, so a row's split -- and with it the exact order of its fp32
// reductions -- depends on that row's own length alone. chunk is a multiple of 16 and at most
// 64 blocks, so one wave holds a chunk's block ids in one register. Both head sizes take the
// largest, 1024 tokens (at D = 128 512-token chunks made the long-context call 4.3% slower once
// the blocks' products moved to the matrix cores).
#ifndef PA_CHUNK_D128
#define PA_CHUNK_D128 1024
#endif
#ifndef PA_CHUNK_D64
#define PA_CHUNK_D64 1024
#endif
static_assert(PA_CHUNK_D128 % 16 == 0 && PA_CHUNK_D128 <= 1024, "chunk: <= 64 blocks");
static_assert(PA_CHUNK_D64 % 16 == 0 && PA_CHUNK_D64 <= 1024, "chunk: <= 64 blocks");
__host__ __device__ inline int chunk_tokens(int head_dim) {
  return head_dim >= 128 ? PA_CHUNK_D128 : PA_CHUNK_D64;
}
__host__ __device__ inline int num_splits(int n, int chunk) {
  return n <= 0 ? 1 : (n + chunk - 1) / chunk;
}

// ---- kernel argument packs ---------------------------------------------------------------
struct AppendArgs {
  int layout, dtype, H_kv, H_q, D;
  int num_blocks, batch_cap, seq_cap, rope_max_pos;
  void* k;
  void* v;
  const float* cos;  // NULL: no RoPE
  const float* sin;
  const int32_t* block_tables;
  int bt_stride;
  const int32_t* positions;
  const int32_t* dest;  // NULL: dest = positions
  const void* k_new;
  const void* v_new;
  const void* q_in;  // NULL: no queries
  void* q_out;
  int batch;
  // per-head RMSNorm before RoPE: weights [D] fp32 (k_norm_w NULL: no normalisation)
  const float* q_norm_w;
  const float* k_norm_w;
  float norm_eps;
};

struct DecodeArgs {
  int layout, dtype, H_kv, H_q, D, n_q;
  int num_blocks;
  int seq_cap;  // padded layout
  const void* k;
  const void* v;
  const void* q;
  long long q_row_stride;  // elements
  const int32_t* block_tables;  // paged
  int bt_stride;
  const int32_t* kv_lens;       // paged
  const int32_t* gap_start;     // padded
  const int32_t* gap_end;       // padded
  int kv_cols;                  // padded
  int batch;
  int max_kv_len;  // host bound: paged max kv_len, padded kv_cols
  int s_max;       // splits of the longest possible row
  float scale;
  float* out;
  float* lse;
  float* part_o;    // [batch][n_q*H_q][s_max][D]
  float* part_lse;  // [batch][n_q*H_q][s_max] (log2 domain)
  int* counter;     // work counter of the persistent decode kernel (0 between calls), or NULL
  int* merge_counts;  // [batch][H_kv] finished splits per (row, KV head) when the split grid
                     // merges its own partials (0 between calls), else NULL
  int ticket_y;     // split grid: first grid row whose workgroups take tickets (0: a plain grid)
  int mq_tiles;     // multi-query path: 16-row query tiles per (row, KV head)
  // block-sparse multi-query path: keep flags [batch][ceil(n_q / 16)][mask_kv_blocks], or NULL
  const uint8_t* block_mask;
  int mask_kv_blocks;
  // append fused into the split kernel (k_new NULL: none). Row b's new key and value go to token
  // index dest[b] (dest NULL: positions[b]) exactly as append_kernel stores them; q holds the
  // un-rotated queries, rotated at positions[b] in registers when cos is set, and the workgroups
  // of split 0 store them to q_out (NULL: not stored).
  const int32_t* positions;
  const int32_t* dest;
  const void* k_new;
  const void* v_new;
  void* q_out;
  const float* cos;  // [rope_max_pos][D/2], or NULL
  const float* sin;
  int rope_max_pos;
  // lockstep step (paged): kv_len of row b is positions[b] + 1 (clamped to max_kv_len) instead of
  // kv_lens[b], and the workgroup of (row b, KV head 0, split 0) writes positions_out[b] =
  // positions[b] + 1
  int kv_from_positions;
  int32_t* positions_out;
};

// Workspace of a decode call (0 bytes when no row can split):
//   [256 B: work counters, 0 before the first call, each call leaves them 0: bytes 0-3 the
//    persistent kernel's, bytes 8-15 the ticketed split grid's] [split partial outputs, fp32]
//   [split partial log-sum-exps, fp32]
constexpr size_t kCounterBytes = 256;
// Workspace of a decode with splits, in this order: the work counters (256 bytes), one
// finished-split count per (row, query head) (a bound of the split grid's per (row, KV head)
// counts, 256-byte rounded; reserved for every call so that partials never land there), the
// partial outputs and their log-sum-exp. The counters lead, at offsets that depend on batch x
// H_q only, so calls of other split counts can share a workspace: every call leaves them at zero.
inline size_t merge_count_bytes(int batch, int H_q) {
  return ((size_t)batch * (size_t)H_q * sizeof(int) + 255) & ~(size_t)255;
}

// c_bytes: the bytes reserved for the finished-split counts, merge_count_bytes(batch, H_q) for a
// caller's workspace, or a fixed reservation that holds the counts of any batch up to a limit (the
// library's own scratch, whose counts then keep their offsets from one call to the next).
inline size_t decode_workspace_bytes(int batch, int n_q, int H_q, int D, int s_max,
                                     size_t c_bytes) {
  if (s_max <= 1) return 0;
  size_t rows = (size_t)batch * (size_t)n_q * (size_t)H_q * (size_t)s_max;
  size_t bytes = kCounterBytes + c_bytes;
  bytes += (rows * (size_t)D * sizeof(float) + 255) & ~(size_t)255;
  bytes += (rows * sizeof(float) + 255) & ~(size_t)255;
  return bytes;
}
inline size_t decode_workspace_bytes(int batch, int n_q, int H_q, int D, int s_max) {
  return decode_workspace_bytes(batch, n_q, H_q, D, s_max, merge_count_bytes(batch, H_q));
}

inline void carve_workspace(void* ws, int batch, int n_q, int H_q, int D, int s_max,
                            size_t c_bytes, int** counter, float** part_o, float** part_lse,
                            int** merge_counts) {
  size_t rows = (size_t)batch * (size_t)n_q * (size_t)H_q * (size_t)s_max;
  size_t o_bytes = (rows * (size_t)D * sizeof(float) + 255) & ~(size_t)255;
  *counter = (int*)ws;
  *merge_counts = n_q == 1 ? (int*)((char*)ws + kCounterBytes) : nullptr;
  *part_o = (float*)((char*)ws + kCounterBytes + c_bytes);
  *part_lse = (float*)((char*)ws + kCounterBytes + c_bytes + o_bytes);
}

// ---- launchers (each returns the hipGetLastError of its launches) -----------------------------
struct TokenizeArgs {
  int H, dh, model_dim, num_blocks;
  void* k;  // bf16 pool
  void* v;
  const float* n_emb;  // [neuron_rows][model_dim]
  const float* t_emb;  // [time_rows][model_dim]
  const float* v_emb;  // [value_rows][model_dim]
  int neuron_rows, time_rows, value_rows;
  const void* w_k;  // bf16 [H * dh][model_dim], packed by launch_pack_projection
  const void* w_v;
  const int32_t* offsets;  // [batch + 1]
  const int32_t* neuron_ids;
  const int32_t* time_bins;
  const int32_t* value_ids;
  int num_events;  // length of the id arrays
  const int32_t* block_tables;
  int bt_stride;
  int batch;
  int max_events;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_tokenize(const TokenizeArgs& a, hipStream_t stream);
int tokenize_max_model_dim();
hipError_t launch_pack_projection(const void* w, void* packed, int out_features, int in_features,
                                  hipStream_t stream);
hipError_t launch_advance(int32_t* positions, int32_t* kv_lens, int32_t* dest, int batch,
                          hipStream_t stream);
// n_q == 1; *merged tells whether the launch also merged the splits (no lse_reduce needed)
hipError_t launch_decode_vector(const DecodeArgs& a, hipStream_t stream, bool* merged);
hipError_t launch_decode_mq(const DecodeArgs& a, hipStream_t stream);      // n_q > 1
hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream);

}  // namespace pa
