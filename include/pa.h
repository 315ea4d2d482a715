/*
 * pa.h -- C ABI of the MI355X (gfx950) paged decode-attention library (libpa.so).
 *
 * The operations, and the passages of the pages they follow:
 *   - a pre-allocated pool of fixed 16-token K/V blocks, reached through per-sequence block tables
 *     ("NeuroGrid releases", v0.7.0 "Paged KV Cache"; "cortex-engine write-up", serving section:
 *     a pre-allocated page pool with a fixed page size);
 *   - appending each row's new key and value at its own position, the key rotated (RoPE,
 *     rotate-half) at that row's logical position before it is stored ("helexa PR #121", commit
 *     "slice 1": per-row RoPE positions; keys stored post-RoPE, so padding is position-inert);
 *   - batched single-token decode attention over the paged cache with GQA and an online softmax
 *     ("NeuroGrid releases", v0.7.0 and v0.6.0 "Flash Decode Attention Kernel"); with several
 *     queries per row it is the ragged multi-query cross-attention of the "cortex-engine
 *     write-up", kernels section, which pa_decode_attention_block_sparse also runs under a
 *     caller's boolean (query block x key block) mask (block-sparse cross-attention);
 *   - the lockstep form over right-padded per-row KV with one padding gap per row
 *     ("helexa PR #121", commit "slice 1": assemble_batch, batch_decode_mask);
 *   - the append with a per-head RMSNorm of the keys (and queries) before the rotation
 *     (pa_append_kv_qk_norm; "NeuroGrid releases", v0.5.0 "LFM2 Hybrid Architecture Support",
 *     Architecture: per-head RMSNorm of Q and K ahead of the rotation);
 *   - advancing a lockstep batch's positions and lengths on the device, so a recorded decode step
 *     can be replayed token after token (pa_advance_lockstep; "NeuroGrid releases", v0.8.0
 *     "CUDA Graphs");
 *   - spike events straight into the pool: the three-table tokenizer fused with the K/V
 *     projection (pa_tokenize_kv; "cortex-engine write-up", model and kernels sections), with
 *     pa_pack_projection to put its weights into the matrix cores' fragment order (a layout of
 *     this library).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns every buffer; the library
 *     allocates nothing, keeps no state beyond a host-side cache of per-kernel occupancy figures
 *     (filled on first use, thread-safe) and never synchronises (except pa_alloc_pool, which
 *     waits for its own table upload). Work is enqueued on `stream` and returns at once.
 *   - Validation of host-side arguments happens before any HIP call; a failed check returns an
 *     error code and launches nothing. A failed launch returns PA_ERR_HIP. No C++ exception
 *     crosses the ABI.
 *   - Device-side contents (lengths, positions, block ids) are preconditions and are not checked
 *     for errors; to keep every access inside the caller's buffers the kernels clamp them (see each
 *     call), which can only turn a broken precondition into a wrong result, never a fault.
 *   - Scores and outputs are computed in fp32. `out` is fp32; `lse` is the natural-log
 *     log-sum-exp of the scaled scores. A row with no valid key yields out = 0 and lse = -inf.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent sizes (negative, not divisible, bound too large, ...) */
  PA_ERR_UNSUPPORTED = 3, /* a valid but unsupported configuration (dtype, head_dim, block size) */
  PA_ERR_CAPACITY = 4,    /* a caller buffer (pool buffer, workspace) is too small */
  PA_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;
typedef enum { PA_PAGED = 0, PA_PADDED = 1 } pa_layout;

/* (host) Shape of a pool. */
typedef struct {
  int32_t layout;        /* pa_layout */
  int32_t dtype;         /* pa_dtype: storage type of K, V and of the queries used with the pool */
  int32_t num_kv_heads;  /* H_kv in [1, 65535] */
  int32_t head_dim;      /* D in {32, 64, 128} */
  int32_t block_size;    /* must be 16 */
  int32_t num_blocks;    /* PA_PAGED: physical blocks (>= 1); ignored for PA_PADDED */
  int32_t batch_cap;     /* PA_PADDED: rows; ignored for PA_PAGED */
  int32_t seq_cap;       /* PA_PADDED: columns per row; ignored for PA_PAGED */
  int32_t rope_max_pos;  /* rows of the RoPE tables; 0 = no RoPE (keys and queries stored as given) */
  double rope_theta;     /* RoPE base theta (> 0 when rope_max_pos > 0) */
} pa_pool_desc;

/* (host) Plain view of a pool carved from caller memory; needs no destructor.
 *   PA_PAGED : k, v are [num_blocks][H_kv][16][D]; token t of a row with block table bt lives at
 *              block bt[t / 16], slot t % 16.
 *   PA_PADDED: k, v are [batch_cap][H_kv][seq_cap][D]; row b's column c lives at [b][.][c].
 *   rope_cos, rope_sin: [rope_max_pos][D / 2] fp32, or NULL without RoPE. */
typedef struct {
  pa_pool_desc desc;
  void* k;
  void* v;
  float* rope_cos;
  float* rope_sin;
  size_t bytes; /* bytes of dev_buf the pool occupies */
} pa_pool;

/* Carve a pool out of one caller-owned device buffer, and fill its RoPE tables.
 *
 * Size query: with dev_buf == NULL, writes the bytes needed to *bytes_needed and returns PA_OK.
 * Otherwise dev_buf (256-byte aligned, dev_buf_bytes long) is split into K, V and the two tables,
 * *out is filled, and the tables are uploaded on `stream`, which the call then synchronises.
 * Table entry [p][i] is cos/sin(p * theta^(-2i/D)), evaluated in fp64 on the host and rounded once
 * to fp32. K/V contents are left as they are (the caller fills or poisons them).
 * Errors: NULL desc / out / bytes_needed -> PA_ERR_NULL; block_size != 16, head_dim not in
 * {32, 64, 128}, unknown dtype or layout -> PA_ERR_UNSUPPORTED; non-positive sizes or theta with a
 * table -> PA_ERR_SHAPE; dev_buf_bytes too small or dev_buf misaligned -> PA_ERR_CAPACITY. */
pa_status pa_alloc_pool(const pa_pool_desc* desc, void* dev_buf, size_t dev_buf_bytes,
                        size_t* bytes_needed /* host */, pa_pool* out /* host */,
                        hipStream_t stream);

/* Append one token per row.
 *
 * Row b (b < batch): the key k_new[b] ([H_kv][D], pool dtype) is rotated at position positions[b]
 * when the pool has RoPE tables -- rotate-half, pairs (i, i + D/2):
 *   r[i] = x[i]*c[i] - x[i+D/2]*s[i],  r[i+D/2] = x[i+D/2]*c[i] + x[i]*s[i]
 * with every product and sum a separate round-to-nearest fp32 operation -- then rounded to the pool
 * dtype (round-to-nearest-even) and written with v_new[b] (copied unchanged) at token index dest[b]:
 * PA_PAGED block block_tables[b * bt_stride + dest[b] / 16], slot dest[b] % 16; PA_PADDED row b,
 * column dest[b]. dest == NULL means dest = positions. q_in/q_out ([batch][num_q_heads][D], pool
 * dtype; both NULL or both set) rotate the queries at the same positions (copied when the pool has
 * no tables). Results are bit-exact and independent of the launch geometry.
 * Preconditions (clamped, not checked): 0 <= positions[b] < rope_max_pos, dest[b] inside the row
 * (< bt_stride*16, or < seq_cap), block ids < num_blocks, b < batch_cap for PA_PADDED.
 * Errors: PA_ERR_NULL for a missing pointer (block_tables is required for PA_PAGED, positions
 * always); PA_ERR_SHAPE for batch < 0 or > 65535, bt_stride < 1, num_q_heads not a positive
 * multiple of H_kv, batch > batch_cap (PA_PADDED). batch == 0 is a no-op. */
pa_status pa_append_kv(const pa_pool* pool, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* positions, const int32_t* dest, const void* k_new,
                       const void* v_new, const void* q_in, void* q_out, int32_t num_q_heads,
                       int32_t batch, hipStream_t stream);

/* Append one token per row, with per-head RMSNorm of the new key (and query) before RoPE
 * ("NeuroGrid releases", v0.5.0 "LFM2 Hybrid Architecture Support", Architecture: a per-head
 * RMSNorm of queries and keys, applied before RoPE).
 *
 * As pa_append_kv, except that every key head x (D elements, fp32 from the pool dtype) -- and every
 * query head when q_in is given -- is first replaced by y_i = (x_i * r) * w_i with
 * r = 1 / sqrt(ss / D + eps), w = k_norm_weight (queries: q_norm_weight), fp32 [D] device arrays.
 * Every operation is a separate correctly rounded fp32 operation, and the sum of squares ss is
 * formed over the rotate-half pairs first, s_i = x_i*x_i + x_{i+D/2}*x_{i+D/2} (i < D/2), then as a
 * pairwise tree of neighbours ((s_0 + s_1), (s_2 + s_3), ..., then those in pairs, ...), so the
 * stored bits are reproducible. The result is then rotated as in pa_append_kv (or, on a pool
 * without RoPE tables, stored as is). Values are not normalised.
 * Errors: as pa_append_kv; PA_ERR_NULL also for k_norm_weight, or q_norm_weight when q_in is
 * given; PA_ERR_SHAPE for eps negative or not finite. */
pa_status pa_append_kv_qk_norm(const pa_pool* pool, const int32_t* block_tables,
                               int32_t bt_stride, const int32_t* positions, const int32_t* dest,
                               const void* k_new, const void* v_new, const void* q_in,
                               void* q_out, int32_t num_q_heads, int32_t batch,
                               const float* q_norm_weight, const float* k_norm_weight, float eps,
                               hipStream_t stream);

/* Paged decode attention.
 *
 * q: [batch][n_q][num_q_heads][D] in the pool dtype; row b starts at element b * q_row_stride
 * (q_row_stride = 0 shares one [n_q][H_q][D] block of queries between all rows). Query head h reads
 * KV head h / G, G = num_q_heads / H_kv. Row b attends over its first kv_lens[b] tokens, gathered
 * through block_tables[b * bt_stride ...]; score = scale * <q, k> (scale finite and >= 0); exact
 * softmax, computed online.
 * out: [batch][n_q][num_q_heads][D] fp32. lse: [batch][n_q][num_q_heads] fp32 or NULL.
 * n_q == 1 is the decode path (vector units; one workgroup per (row, KV head, split); long rows are
 * split into chunks whose partial results are merged by log-sum-exp: by the split kernel
 * itself when no row has more than 16 chunks, else by a second kernel). n_q > 1 is the
 * multi-query path (matrix cores). The split of a row depends on its own kv_len only, so a row's
 * result does not depend on the rest of the batch.
 * Workspace: with workspace_needed != NULL the call only writes the bytes it needs for these
 * arguments there and launches nothing; otherwise workspace must hold that many bytes and be
 * 256-byte aligned (it may be NULL when none are needed). A workspace must be zero-filled before
 * its first use: it starts with counters that every call leaves at zero again, the work counters of
 * the split kernels (256 bytes) and one finished-split count per (row, query head) (4 * batch *
 * num_q_heads bytes, rounded up to 256), with the partial results after them. Calls may share a
 * workspace while batch * num_q_heads stays the same (their split counts may differ); after a
 * change, zero-fill it again (a smaller call's partials overwrite a larger one's counts). A call
 * that returns PA_ERR_HIP may have stopped with its counters raised: zero-fill the workspace
 * again before the next call uses it. Calls that overlap in time (other streams) need workspaces
 * of their own. max_kv_len is a host upper bound of kv_lens (<= bt_stride * 16).
 * Preconditions (clamped, not checked): 0 <= kv_lens[b] <= max_kv_len; block ids < num_blocks.
 * Errors: PA_ERR_NULL (pool, q, block_tables, kv_lens, out); PA_ERR_SHAPE (batch < 0 or > 65535,
 * n_q < 1, num_q_heads not a positive multiple of H_kv, max_kv_len < 0 or > bt_stride * 16, more
 * than 65535 splits for max_kv_len, layout not PA_PAGED, scale negative or not finite, q not
 * 16-byte aligned or q_row_stride not a multiple of 16 bytes); PA_ERR_UNSUPPORTED (n_q == 1 with G
 * not in {1, 2, 4, 8}; n_q > 1 with an fp32 pool); PA_ERR_CAPACITY (workspace too small or not
 * 256-byte aligned). batch == 0 is a no-op. */
pa_status pa_decode_attention(const pa_pool* pool, const void* q, int64_t q_row_stride,
                              int32_t n_q, int32_t num_q_heads, const int32_t* block_tables,
                              int32_t bt_stride, const int32_t* kv_lens, int32_t batch,
                              int32_t max_kv_len, float scale, void* workspace,
                              size_t workspace_bytes, size_t* workspace_needed /* host */,
                              float* out, float* lse, hipStream_t stream);

/* Scratch of pa_decode_attention_noalloc: its size per device, and the most (row, query head)
 * pairs of one call whose finished-split counts it reserves room for. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
#define PA_NOALLOC_MAX_ROW_HEADS 16384

/* pa_decode_attention for callers that cannot allocate device memory: code under stream or graph
 * capture, tight serving loops, harnesses that forbid allocation. Same arguments, results and
 * errors as pa_decode_attention, without the workspace: the split partials go to the library's
 * own scratch, one PA_NOALLOC_SCRATCH_BYTES array per device, allocated with the library's code on
 * that device and held until the process ends. The call allocates and frees nothing.
 * Limits: a call needing more scratch than PA_NOALLOC_SCRATCH_BYTES (for the split rows: 256 +
 * 4 * PA_NOALLOC_MAX_ROW_HEADS bytes of counters, then batch * n_q * num_q_heads * splits * (D + 1)
 * fp32 partials, each part 256-byte rounded), or with batch * num_q_heads > PA_NOALLOC_MAX_ROW_HEADS
 * when rows can split, returns PA_ERR_CAPACITY before any HIP call. B=128 rows of up to 8192
 * tokens with 32 query heads at D = 64 use 8.5 MB; 4 rows of up to 131072 tokens at D = 128,
 * 14.5 MB.
 * Every call on a device shares that device's scratch, and each call leaves in it only zeroed
 * counters and its own partials: calls that overlap in time on one device (other streams, other
 * threads) race and must not be issued. The first call on a device clears the counters with a
 * small kernel on `stream` (and so does the first call after a failed launch); under stream
 * capture that clear is recorded too. Calls without split rows (every kv_len within one chunk)
 * and multi-query calls use no scratch. */
pa_status pa_decode_attention_noalloc(const pa_pool* pool, const void* q, int64_t q_row_stride,
                                      int32_t n_q, int32_t num_q_heads,
                                      const int32_t* block_tables, int32_t bt_stride,
                                      const int32_t* kv_lens, int32_t batch, int32_t max_kv_len,
                                      float scale, float* out, float* lse, hipStream_t stream);

/* Projection weights in matrix-core fragment order, for pa_tokenize_kv (a layout of this library,
 * not of the pages: one A-operand fragment of the 16x16x32 bf16 matrix-core product is 64 lanes x
 * 16 contiguous bytes, so the tokenizer reads each with one coalesced 1 KB load).
 * w: bf16 [out_features][in_features] (a linear layer's weight), device. packed: device, as many
 * bytes, must not overlap w; on return
 *   packed[((tile * (in_features / 32) + kc) * 64 + lane) * 8 + j]
 *     = w[16 tile + lane % 16][32 kc + 8 (lane / 16) + j]
 * for tile < out_features / 16, kc < in_features / 32, lane < 64, j < 8 (a permutation: values
 * are copied bit for bit). Asynchronous on stream.
 * Errors: PA_ERR_NULL; PA_ERR_SHAPE (out_features not a positive multiple of 16, in_features not a
 * positive multiple of 32, a pointer not 16-byte aligned, overlapping buffers). */
pa_status pa_pack_projection(const void* w, int32_t out_features, int32_t in_features,
                             void* packed, hipStream_t stream);

/* Spike tokens straight into the paged pool: the fused three-table tokenizer and K/V projection
 * ("cortex-engine write-up", model section and kernels section, fused spike tokenizer: each spike
 * event (neuron_id, time_bin, value) is the sum of three embedding-table rows; "NeuroGrid
 * releases", v0.7.0: tokens stored through per-sequence block tables).
 *
 * Row b's tokens are its events offsets[b] .. offsets[b+1] - 1 (int32 CSR offsets [batch + 1] into
 * neuron_ids / time_bins / value_ids, device, each num_events long), at most max_events of them
 * (more are ignored). Offsets are clamped into [0, num_events].
 * Token t (0-based within the row) has the embedding x = (neuron_table[neuron_ids[e]] +
 * time_table[time_bins[e]]) + value_table[value_ids[e]] (fp32 tables [rows][model_dim], each sum
 * one fp32 operation; ids clamped into their tables), rounded to bf16. Its key is x . W_k^T and
 * its value x . W_v^T (bf16 weights [H_kv * head_dim][model_dim], the layout of a linear layer's
 * weight; products summed in fp32 on the matrix cores, in an unspecified order), rounded to bf16
 * and stored as heads of head_dim at slot (block_tables[b * bt_stride + t / 16], t % 16). Only the
 * rows' token slots are written. The embeddings never reach memory.
 * w_k_packed / w_v_packed are W_k and W_v as pa_pack_projection leaves them (device, H_kv *
 * head_dim * model_dim bf16 each); pack once, reuse for every call.
 * Requirements: a PA_PAGED bf16 pool; model_dim a multiple of 32 in [32, 512]; tables and packed
 * weights 16-byte aligned; max_events <= bt_stride * 16.
 * Errors: PA_ERR_NULL (any pointer); PA_ERR_UNSUPPORTED (fp32 pool, model_dim out of range);
 * PA_ERR_SHAPE (layout not PA_PAGED, table rows < 1, batch < 0 or > 65535, bt_stride < 1,
 * num_events < 0, max_events < 0 or > bt_stride * 16, misaligned tables or weights). batch == 0,
 * num_events == 0 or max_events == 0 is a no-op. */
pa_status pa_tokenize_kv(const pa_pool* pool, const float* neuron_table, int32_t neuron_rows,
                         const float* time_table, int32_t time_rows, const float* value_table,
                         int32_t value_rows, int32_t model_dim, const void* w_k_packed,
                         const void* w_v_packed, const int32_t* offsets, const int32_t* neuron_ids,
                         const int32_t* time_bins, const int32_t* value_ids,
                         int32_t num_events, const int32_t* block_tables, int32_t bt_stride,
                         int32_t batch, int32_t max_events, hipStream_t stream);

/* Advance a lockstep batch by one token, on the device ("NeuroGrid releases", v0.8.0: the whole
 * decode step replayed as a graph, with position and kv_len read from device buffers and an
 * add-one kernel computing kv_len = position + 1 on the GPU).
 *
 * For b < batch: positions[b] += 1; then, when kv_lens != NULL, kv_lens[b] = positions[b] + 1;
 * when dest != NULL, dest[b] += 1 (all int32, device). With it a captured step (append at the
 * positions, decode over kv_lens, advance) replays with no host work between tokens; the caller
 * keeps the block tables filled for the positions ahead. Positions must stay below 2^31 - 2.
 * Errors: PA_ERR_NULL (positions); PA_ERR_SHAPE (batch < 0). batch == 0 is a no-op. */
pa_status pa_advance_lockstep(int32_t* positions, int32_t* kv_lens, int32_t* dest, int32_t batch,
                              hipStream_t stream);

/* Block-sparse multi-query decode attention over the paged cache ("cortex-engine write-up",
 * kernels section, block-sparse cross-attention: a boolean tile mask computed outside the kernel;
 * tiles whose mask is false are skipped; a query left with no key gives zeros, not NaN).
 *
 * As pa_decode_attention (same q, q_row_stride, block_tables, kv_lens, out and lse contracts),
 * plus block_mask: uint8 [batch][ceil(n_q / 16)][mask_kv_blocks] (device). Query i of row b
 * attends exactly to the keys of the 16-token blocks j (tokens 16j .. 16j + 15, j < ceil(kv_len /
 * 16)) with block_mask[b][i / 16][j] != 0; a query with no such key gets out = 0 and lse = -inf.
 * mask_kv_blocks is the row stride of the mask, >= ceil(max_kv_len / 16). Every query head of a
 * query shares the query's mask. Runs on the matrix cores for any n_q >= 1; a row is never split,
 * so no workspace is needed. Dropped blocks are neither read nor computed.
 * Errors: PA_ERR_NULL (pool, q, block_tables, kv_lens, block_mask, out); PA_ERR_SHAPE (as for
 * pa_decode_attention, and mask_kv_blocks < max(1, ceil(max_kv_len / 16))); PA_ERR_UNSUPPORTED
 * (fp32 pool). batch == 0 is a no-op. */
pa_status pa_decode_attention_block_sparse(const pa_pool* pool, const void* q,
                                           int64_t q_row_stride, int32_t n_q, int32_t num_q_heads,
                                           const int32_t* block_tables, int32_t bt_stride,
                                           const int32_t* kv_lens, int32_t batch,
                                           int32_t max_kv_len, float scale,
                                           const uint8_t* block_mask, int32_t mask_kv_blocks,
                                           float* out, float* lse, hipStream_t stream);

/* Lockstep decode over right-padded KV (PA_PADDED pool).
 *
 * q: [batch][num_q_heads][D] in the pool dtype. Row b's valid columns are
 * [0, gap_start[b]) and [gap_end[b], kv_cols); the gap in between is skipped (never read), which
 * equals an additive -inf mask on it. gap_start == gap_end means no gap. out/lse as for
 * pa_decode_attention; the same split rule applies to the row's count of valid columns.
 * Workspace as for pa_decode_attention.
 * Preconditions (clamped, not checked): 0 <= gap_start[b] <= gap_end[b] <= kv_cols.
 * Errors: PA_ERR_NULL (pool, q, gap_start, gap_end, out); PA_ERR_SHAPE (batch < 0, > batch_cap
 * or > 65535, kv_cols < 0 or > seq_cap, more than 65535 splits for kv_cols, num_q_heads not a positive multiple of H_kv, layout not PA_PADDED,
 * scale negative or not finite, q not 16-byte aligned);
 * PA_ERR_UNSUPPORTED (G not in {1, 2, 4, 8}); PA_ERR_CAPACITY (workspace too small or not
 * 256-byte aligned). */
pa_status pa_decode_attention_padded(const pa_pool* padded_pool, const void* q,
                                     int32_t num_q_heads, int32_t batch, const int32_t* gap_start,
                                     const int32_t* gap_end, int32_t kv_cols, float scale,
                                     void* workspace, size_t workspace_bytes,
                                     size_t* workspace_needed /* host */, float* out, float* lse,
                                     hipStream_t stream);

/* Append and decode in one call: pa_append_kv followed by pa_decode_attention on the rotated
 * queries, with the append folded into the decode kernel (helexa PR #121, commit
 * "slice 1": per-row positions, keys stored post-RoPE; "NeuroGrid releases", v0.7.0: block-table
 * slots; v0.6.0: the decode). One launch instead of two.
 *
 * Row b's new key k_new[b] and value v_new[b] ([H_kv][D], pool dtype) are stored at token index
 * dest[b] (NULL: positions[b]) exactly as pa_append_kv stores them (same rotation, rounding,
 * clamping), and the row then attends over its first kv_lens[b] tokens, which see the new token
 * when dest[b] < kv_lens[b]. q: [batch][num_q_heads][D], pool dtype, the queries before rotation;
 * on a pool with RoPE tables they are rotated at positions[b] exactly as pa_append_kv rotates
 * them and the result is stored to q_out (same shape, required), otherwise q is used as given and
 * copied to q_out when q_out is not NULL. q_out must not overlap q. Results (pool bits, q_out,
 * out, lse) equal those of the two separate calls bit for bit.
 * Workspace, out, lse, kv_lens, max_kv_len and block tables as for pa_decode_attention (n_q = 1).
 * Preconditions (clamped, not checked): as for both calls; in addition no row reads another row's
 * destination slot (destination slots are private to their rows).
 * Errors: those of pa_decode_attention with n_q = 1 and q_row_stride = num_q_heads * D; then
 * PA_ERR_NULL (positions, k_new, v_new; q_out on a pool with RoPE tables); PA_ERR_SHAPE (k_new,
 * v_new or q_out not 16-byte aligned, q_out overlapping q). */
pa_status pa_append_decode_attention(const pa_pool* pool, const int32_t* block_tables,
                                     int32_t bt_stride, const int32_t* positions,
                                     const int32_t* dest, const void* k_new, const void* v_new,
                                     const void* q, void* q_out, int32_t num_q_heads,
                                     const int32_t* kv_lens, int32_t batch, int32_t max_kv_len,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     size_t* workspace_needed /* host */, float* out, float* lse,
                                     hipStream_t stream);

/* One lockstep decode step in one launch: pa_append_decode_attention with kv_len = position + 1
 * taken on the device, and the positions of the next step written out ("NeuroGrid releases",
 * v0.8.0 "CUDA Graphs": position and kv_len read from device buffers, kv_len = position + 1
 * computed on the GPU, so a recorded step replays token after token with no host work).
 *
 * Row b's new key and value are stored at token index positions[b] (rotated there when the pool
 * has RoPE tables), and the row attends over its first kv_len = positions[b] + 1 tokens (clamped
 * into [0, max_kv_len]), exactly as pa_append_decode_attention does with dest = NULL and
 * kv_lens[b] = positions[b] + 1, bit for bit. In the same launch positions_out[b] =
 * positions[b] + 1 (int32, device, [batch], must not overlap positions): the next step reads
 * positions_out, so two buffers alternate from step to step and the step needs no second kernel.
 * Other arguments, the workspace and the errors as for pa_append_decode_attention; in addition
 * PA_ERR_NULL (positions_out) and PA_ERR_SHAPE (positions_out overlapping positions). Positions
 * must stay below 2^31 - 2. */
pa_status pa_lockstep_decode_step(const pa_pool* pool, const int32_t* block_tables,
                                  int32_t bt_stride, const int32_t* positions,
                                  int32_t* positions_out, const void* k_new, const void* v_new,
                                  const void* q, void* q_out, int32_t num_q_heads, int32_t batch,
                                  int32_t max_kv_len, float scale, void* workspace,
                                  size_t workspace_bytes, size_t* workspace_needed /* host */,
                                  float* out, float* lse, hipStream_t stream);

/* The lockstep form of pa_append_decode_attention over a PA_PADDED pool: pa_append_kv (new token
 * at column dest[b], NULL: positions[b]) followed by pa_decode_attention_padded, in one launch.
 * Arguments and results as for those two calls and pa_append_decode_attention; a destination
 * column inside the row's gap or at or past kv_cols is written but not attended to.
 * Errors: those of pa_decode_attention_padded, then those of pa_append_decode_attention's
 * append half. */
pa_status pa_append_decode_attention_padded(const pa_pool* padded_pool, const int32_t* positions,
                                            const int32_t* dest, const void* k_new,
                                            const void* v_new, const void* q, void* q_out,
                                            int32_t num_q_heads, const int32_t* gap_start,
                                            const int32_t* gap_end, int32_t kv_cols,
                                            int32_t batch, float scale, void* workspace,
                                            size_t workspace_bytes,
                                            size_t* workspace_needed /* host */, float* out,
                                            float* lse, hipStream_t stream);

/* Merge partial attention results computed over disjoint key sets (the step after an all-gather
 * when one row's keys are split across GPUs). The pages never split a row; this is the log-sum-exp
 * merge of this library's own split-K design, the algebra pa_decode_attention applies to the
 * chunks of a long row.
 *
 * out_parts: fp32 [num_parts][n][head_dim], each part's normalised output for n (row, query head)
 * pairs; lse_parts: fp32 [num_parts][n], each part's log-sum-exp (natural log, -inf for a part
 * with no keys) -- what pa_decode_attention writes for each part's keys. For every pair:
 *   M = max_p lse_p,  w_p = exp(lse_p - M),  out = sum_p w_p out_p / sum_p w_p,
 *   lse = M + log(sum_p w_p)   (fp32, parts summed in index order)
 * out: fp32 [n][head_dim]; lse: fp32 [n] or NULL. Every part empty gives out = 0, lse = -inf.
 * Device pointers; out must not overlap out_parts. Asynchronous on stream; no workspace.
 * Errors: PA_ERR_NULL (out_parts, lse_parts, out); PA_ERR_UNSUPPORTED (head_dim not in
 * {32, 64, 128}); PA_ERR_SHAPE (num_parts < 1 or > 65535, n < 0 or > 2^34, out overlapping
 * out_parts). n == 0 is a no-op. */
pa_status pa_lse_merge(const float* out_parts, const float* lse_parts, int32_t num_parts,
                       int64_t n, int32_t head_dim, float* out, float* lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
