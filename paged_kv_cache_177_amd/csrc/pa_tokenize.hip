// Fused spike tokenizer + K/V projection into the paged pool, for gfx950.
//
// What it computes ("cortex-engine write-up", model section and kernels section, fused spike
// tokenizer): each spike event (neuron id, time bin, value) of a row becomes a token whose
// embedding is the sum of three table rows, x = (n_emb[neuron] + t_emb[bin]) + v_emb[value] in
// fp32; its key and value are x . W_k^T and x . W_v^T, split into the pool's heads and stored at
// the token's slot through the row's block table ("NeuroGrid releases", v0.7.0 "Paged KV Cache").
// The embeddings never go to HBM: they are built in LDS and fed to the matrix cores.
//
// Mapping: one workgroup (4 waves) per kTB consecutive 16-token blocks of one row.
//   1. The blocks' event ids go to LDS; each thread then builds 16 consecutive dims of one
//      token's embedding from the three tables (fp32, float4 loads), rounds them to bf16 (the
//      matrix-core input) and parks them in LDS: X [16 kTB][Dm].
//   2. The output columns (H * dh of K, then as many of V) are cut into 16-wide tiles dealt to
//      the waves. Per tile and per 32-wide slice of Dm, a wave loads the slice of W once (B
//      operand: output column lane % 16, 8 consecutive inputs) and applies it to the kTB token
//      tiles (A operand from LDS: token lane % 16, the same 8 inputs): v_mfma_f32_16x16x32_bf16
//      with fp32 accumulation.
//   3. Lane l of an accumulator holds tokens 4 (l / 16) .. + 3 of output column l % 16: each is
//      rounded to bf16 and stored at [block][head = col / dh][slot][col % dh].
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTB = 2;           // 16-token blocks per workgroup
constexpr int kTok = 16 * kTB;   // tokens per workgroup
constexpr int kWaves = 4;
constexpr int kMaxDm = 512;      // LDS holds X [kTok][kMaxDm + 8] bf16

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__global__ __launch_bounds__(64 * kWaves) void tokenize_kv_kernel(const TokenizeArgs a) {
  __shared__ int s_ids[kTok][3];
  __shared__ __attribute__((aligned(16))) unsigned short s_x[kTok][kMaxDm + 8];
  const int row = (int)blockIdx.y;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Dm = a.model_dim;
  // the row's events, clamped into the id arrays [0, num_events)
  const int e0 = clampi(a.offsets[row], 0, a.num_events);
  const int e1 = clampi(a.offsets[row + 1], e0, a.num_events);
  const int n = e1 - e0 < a.max_events ? e1 - e0 : a.max_events;
  const int t0 = (int)blockIdx.x * kTok;  // first token of this workgroup in the row
  if (t0 >= n) return;
  const int nt = n - t0 < kTok ? n - t0 : kTok;

  // 1. event ids of the tokens, then their bf16 embeddings
  if (tid < kTok) {
    int nid = 0, bin = 0, val = 0;
    if (tid < nt) {
      const int e = e0 + t0 + tid;
      nid = clampi(a.neuron_ids[e], 0, a.neuron_rows - 1);
      bin = clampi(a.time_bins[e], 0, a.time_rows - 1);
      val = clampi(a.value_ids[e], 0, a.value_rows - 1);
    }
    s_ids[tid][0] = nid;
    s_ids[tid][1] = bin;
    s_ids[tid][2] = val;
  }
  __syncthreads();
  {
    // each thread: 16 consecutive dims (d0 .. d0 + 15) of one token; Dm / 16 threads per token
    const int per_tok = Dm / 16;
    for (int w = tid; w < kTok * per_tok; w += 64 * kWaves) {
      const int t = w / per_tok;
      const int d0 = (w % per_tok) * 16;
      unsigned short* xs = &s_x[t][d0];
      if (t < nt) {
        const float4* pn = reinterpret_cast<const float4*>(a.n_emb + (size_t)s_ids[t][0] * Dm + d0);
        const float4* pt = reinterpret_cast<const float4*>(a.t_emb + (size_t)s_ids[t][1] * Dm + d0);
        const float4* pv = reinterpret_cast<const float4*>(a.v_emb + (size_t)s_ids[t][2] * Dm + d0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 x = pn[c], y = pt[c], z = pv[c];
          // (n + t) + v, each sum one fp32 operation
          const float r0 = (x.x + y.x) + z.x, r1 = (x.y + y.y) + z.y;
          const float r2 = (x.z + y.z) + z.z, r3 = (x.w + y.w) + z.w;
          xs[4 * c + 0] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(r0));
          xs[4 * c + 1] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(r1));
          xs[4 * c + 2] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(r2));
          xs[4 * c + 3] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(r3));
        }
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) xs[c] = 0;
      }
    }
  }
  __syncthreads();

  // 2. the projection, 16 output columns at a time
  const int N = a.H * a.dh;  // columns of K (and of V)
  const int tiles = 2 * N / 16;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // the pool block of each 16-token sub-block that holds tokens (the table row has bt_stride
  // entries and t0 + 16 b < n <= bt_stride * 16 for those)
  int bids[kTB];
#pragma unroll
  for (int b = 0; b < kTB; ++b)
    bids[b] = 16 * b < nt ? clampi(a.block_tables[(size_t)row * a.bt_stride + (t0 >> 4) + b], 0,
                                   a.num_blocks - 1)
                          : 0;
  for (int tile = wave; tile < tiles; tile += kWaves) {
    const bool is_v = tile * 16 >= N;
    const int c0 = tile * 16 - (is_v ? N : 0);  // first column of the tile inside K or V
    const __bf16* w = reinterpret_cast<const __bf16*>(is_v ? a.w_v : a.w_k) +
                      (size_t)(c0 + col) * Dm + 8 * grp;
    f32x4_t acc[kTB];
#pragma unroll
    for (int b = 0; b < kTB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < Dm; kk += 32) {
      const u32x4_t wb = *reinterpret_cast<const u32x4_t*>(w + kk);
#pragma unroll
      for (int b = 0; b < kTB; ++b) {
        const u32x4_t xa = *reinterpret_cast<const u32x4_t*>(&s_x[16 * b + col][kk + 8 * grp]);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                         __builtin_bit_cast(bf16x8_t, wb), acc[b],
                                                         0, 0, 0);
      }
    }
    // 3. store: lane holds tokens 16 b + 4 grp + j of column c0 + col
    const int c = c0 + col;
    const int head = c / a.dh;
    const int dim = c % a.dh;
    __bf16* pool = reinterpret_cast<__bf16*>(is_v ? a.v : a.k);
#pragma unroll
    for (int b = 0; b < kTB; ++b) {
      // tokens of sub-block b live in the row's block (t0 >> 4) + b
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * b + 4 * grp + j;
        if (t < nt)
          pool[(((size_t)bids[b] * a.H + head) * kBlock + (t & 15)) * a.dh + dim] =
              static_cast<__bf16>(acc[b][j]);
      }
    }
  }
}

}  // namespace

int tokenize_max_model_dim() { return kMaxDm; }

hipError_t launch_tokenize(const TokenizeArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.max_events <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.max_events + kTok - 1) / kTok), (unsigned)a.batch);
  hipLaunchKernelGGL(tokenize_kv_kernel, grid, dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
