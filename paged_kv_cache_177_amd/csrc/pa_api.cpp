// C-ABI layer of libpa.so: host-side validation, pool carving, RoPE tables, launch dispatch.
// Every check runs before the first HIP call, so the error paths work without a GPU.
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"
#include "pa_merge.h"

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int elem_size(int dtype) { return dtype == PA_F32 ? 4 : 2; }

pa_status check_desc(const pa_pool_desc* d) {
  if (d == nullptr) return PA_ERR_NULL;
  if (d->layout != PA_PAGED && d->layout != PA_PADDED) return PA_ERR_UNSUPPORTED;
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (d->block_size != pa::kBlock) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->num_kv_heads < 1 || d->num_kv_heads > pa::kMaxGridYZ) return PA_ERR_SHAPE;
  if (d->layout == PA_PAGED && d->num_blocks < 1) return PA_ERR_SHAPE;
  if (d->layout == PA_PADDED && (d->batch_cap < 1 || d->seq_cap < 1)) return PA_ERR_SHAPE;
  if (d->rope_max_pos < 0) return PA_ERR_SHAPE;
  if (d->rope_max_pos > 0 && !(d->rope_theta > 0.0)) return PA_ERR_SHAPE;
  return PA_OK;
}

size_t kv_bytes(const pa_pool_desc* d) {
  const size_t per_token = (size_t)d->num_kv_heads * (size_t)d->head_dim * elem_size(d->dtype);
  const size_t tokens = d->layout == PA_PAGED ? (size_t)d->num_blocks * pa::kBlock
                                              : (size_t)d->batch_cap * (size_t)d->seq_cap;
  return align256(tokens * per_token);
}

size_t table_bytes(const pa_pool_desc* d) {
  return align256((size_t)d->rope_max_pos * (size_t)(d->head_dim / 2) * sizeof(float));
}

// A pool handed back by the caller must still describe a consistent, carved pool.
pa_status check_pool(const pa_pool* p) {
  if (p == nullptr) return PA_ERR_NULL;
  pa_status s = check_desc(&p->desc);
  if (s != PA_OK) return s;
  if (p->k == nullptr || p->v == nullptr) return PA_ERR_NULL;
  if (p->desc.rope_max_pos > 0 && (p->rope_cos == nullptr || p->rope_sin == nullptr))
    return PA_ERR_NULL;
  return PA_OK;
}

// q rows must keep the kernels' 16-byte vector loads aligned.
bool q_aligned(const void* q, long long row_stride, int dtype) {
  const long long per16 = 16 / elem_size(dtype);
  return ((uintptr_t)q % 16) == 0 && (row_stride % per16) == 0;
}

// cos/sin are called through volatile pointers so that the compiler cannot fuse them into a
// sincos call or fold them: every entry is the host libm's own cos(a), sin(a).
double (*volatile g_cos)(double) = std::cos;
double (*volatile g_sin)(double) = std::sin;
double (*volatile g_pow)(double, double) = std::pow;

pa_status map_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

}  // namespace

extern "C" pa_status pa_alloc_pool(const pa_pool_desc* desc, void* dev_buf, size_t dev_buf_bytes,
                                   size_t* bytes_needed, pa_pool* out, hipStream_t stream) {
  if (desc == nullptr) return PA_ERR_NULL;
  pa_status s = check_desc(desc);
  if (s != PA_OK) return s;
  const size_t kvb = kv_bytes(desc);
  const size_t tb = table_bytes(desc);
  const size_t need = 2 * kvb + 2 * tb;
  if (dev_buf == nullptr) {
    if (bytes_needed == nullptr) return PA_ERR_NULL;
    *bytes_needed = need;
    return PA_OK;
  }
  if (out == nullptr) return PA_ERR_NULL;
  if (dev_buf_bytes < need || ((uintptr_t)dev_buf % 256) != 0) return PA_ERR_CAPACITY;
  if (bytes_needed != nullptr) *bytes_needed = need;

  pa_pool p;
  std::memset(&p, 0, sizeof(p));
  p.desc = *desc;
  char* base = static_cast<char*>(dev_buf);
  p.k = base;
  p.v = base + kvb;
  p.rope_cos = desc->rope_max_pos > 0 ? reinterpret_cast<float*>(base + 2 * kvb) : nullptr;
  p.rope_sin = desc->rope_max_pos > 0 ? reinterpret_cast<float*>(base + 2 * kvb + tb) : nullptr;
  p.bytes = need;

  if (desc->rope_max_pos > 0) {
    // Entry [pos][i] = cos/sin(pos * theta^(-2i/D)); frequency and angle in fp64, one rounding to
    // fp32 (helexa PR #121, commit "slice 1": cos/sin gathered per position, rotate-half halves).
    const int half = desc->head_dim / 2;
    const size_t n = (size_t)desc->rope_max_pos * half;
    std::vector<float> cs(n), sn(n);
    for (int i = 0; i < half; ++i) {
      const double inv = g_pow(desc->rope_theta, -2.0 * i / desc->head_dim);
      for (int pos = 0; pos < desc->rope_max_pos; ++pos) {
        const double ang = (double)pos * inv;
        cs[(size_t)pos * half + i] = (float)g_cos(ang);
        sn[(size_t)pos * half + i] = (float)g_sin(ang);
      }
    }
    hipError_t e = hipMemcpyAsync(p.rope_cos, cs.data(), n * sizeof(float),
                                  hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(p.rope_sin, sn.data(), n * sizeof(float), hipMemcpyHostToDevice,
                         stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  *out = p;
  return PA_OK;
}

namespace {

// Validation and argument pack of an append (pa_append_kv, pa_append_kv_qk_norm, and the
// fused-append call where it appends first).
pa_status append_prepare(const pa_pool* pool, const int32_t* block_tables, int32_t bt_stride,
                         const int32_t* positions, const int32_t* dest, const void* k_new,
                         const void* v_new, const void* q_in, void* q_out, int32_t num_q_heads,
                         int32_t batch, const float* q_norm_w, const float* k_norm_w,
                         float norm_eps, pa::AppendArgs* out) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  const pa_pool_desc& d = pool->desc;
  if (positions == nullptr || k_new == nullptr || v_new == nullptr) return PA_ERR_NULL;
  if ((q_in == nullptr) != (q_out == nullptr)) return PA_ERR_NULL;
  if (d.layout == PA_PAGED && block_tables == nullptr) return PA_ERR_NULL;
  if (batch < 0 || batch > pa::kMaxGridYZ) return PA_ERR_SHAPE;
  if (d.layout == PA_PAGED && bt_stride < 1) return PA_ERR_SHAPE;
  if (d.layout == PA_PADDED && batch > d.batch_cap) return PA_ERR_SHAPE;
  if (q_in != nullptr && (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0))
    return PA_ERR_SHAPE;

  pa::AppendArgs& a = *out;
  std::memset(&a, 0, sizeof(a));
  a.layout = d.layout;
  a.dtype = d.dtype;
  a.H_kv = d.num_kv_heads;
  a.H_q = q_in != nullptr ? num_q_heads : 0;
  a.D = d.head_dim;
  a.num_blocks = d.num_blocks;
  a.batch_cap = d.batch_cap;
  a.seq_cap = d.seq_cap;
  a.rope_max_pos = d.rope_max_pos;
  a.k = pool->k;
  a.v = pool->v;
  a.cos = d.rope_max_pos > 0 ? pool->rope_cos : nullptr;
  a.sin = d.rope_max_pos > 0 ? pool->rope_sin : nullptr;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.positions = positions;
  a.dest = dest;
  a.k_new = k_new;
  a.v_new = v_new;
  a.q_in = q_in;
  a.q_out = q_out;
  a.batch = batch;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.norm_eps = norm_eps;
  return PA_OK;
}

pa_status append_common(const pa_pool* pool, const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* positions, const int32_t* dest, const void* k_new,
                        const void* v_new, const void* q_in, void* q_out, int32_t num_q_heads,
                        int32_t batch, const float* q_norm_w, const float* k_norm_w,
                        float norm_eps, hipStream_t stream) {
  pa::AppendArgs a;
  const pa_status s = append_prepare(pool, block_tables, bt_stride, positions, dest, k_new, v_new,
                                     q_in, q_out, num_q_heads, batch, q_norm_w, k_norm_w,
                                     norm_eps, &a);
  if (s != PA_OK || batch == 0) return s;
  return map_hip(pa::launch_append(a, stream));
}

}  // namespace

extern "C" pa_status pa_append_kv(const pa_pool* pool, const int32_t* block_tables,
                                  int32_t bt_stride, const int32_t* positions, const int32_t* dest,
                                  const void* k_new, const void* v_new, const void* q_in,
                                  void* q_out, int32_t num_q_heads, int32_t batch,
                                  hipStream_t stream) {
  return append_common(pool, block_tables, bt_stride, positions, dest, k_new, v_new, q_in, q_out,
                       num_q_heads, batch, nullptr, nullptr, 0.f, stream);
}

extern "C" pa_status pa_append_kv_qk_norm(const pa_pool* pool, const int32_t* block_tables,
                                          int32_t bt_stride, const int32_t* positions,
                                          const int32_t* dest, const void* k_new,
                                          const void* v_new, const void* q_in, void* q_out,
                                          int32_t num_q_heads, int32_t batch,
                                          const float* q_norm_weight, const float* k_norm_weight,
                                          float eps, hipStream_t stream) {
  if (k_norm_weight == nullptr || (q_in != nullptr && q_norm_weight == nullptr))
    return PA_ERR_NULL;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return PA_ERR_SHAPE;
  return append_common(pool, block_tables, bt_stride, positions, dest, k_new, v_new, q_in, q_out,
                       num_q_heads, batch, q_norm_weight, k_norm_weight, eps, stream);
}

namespace {

// Validation and argument pack of the paged decode (pa_decode_attention and the fused-append
// call); *need is the workspace the call requires.
pa_status paged_decode_prepare(const pa_pool* pool, const void* q, int64_t q_row_stride,
                               int32_t n_q, int32_t num_q_heads, const int32_t* block_tables,
                               int32_t bt_stride, const int32_t* kv_lens, int32_t batch,
                               int32_t max_kv_len, float scale, float* out, float* lse,
                               pa::DecodeArgs* a, size_t* need) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  const pa_pool_desc& d = pool->desc;
  if (d.layout != PA_PAGED) return PA_ERR_SHAPE;
  if (q == nullptr || block_tables == nullptr || kv_lens == nullptr || out == nullptr)
    return PA_ERR_NULL;
  if (batch < 0 || batch > pa::kMaxGridYZ || n_q < 1 || bt_stride < 1 || max_kv_len < 0 ||
      q_row_stride < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_kv_len > (int64_t)bt_stride * pa::kBlock) return PA_ERR_SHAPE;
  const int G = num_q_heads / d.num_kv_heads;
  if (n_q == 1 && G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  if (n_q > 1 && d.dtype != PA_BF16) return PA_ERR_UNSUPPORTED;  // matrix-core path: bf16 only
  if (!q_aligned(q, q_row_stride, d.dtype)) return PA_ERR_SHAPE;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;

  const int s_max = n_q == 1 ? pa::num_splits(max_kv_len, pa::chunk_tokens(d.head_dim)) : 1;
  if (s_max > pa::kMaxGridYZ) return PA_ERR_SHAPE;
  *need = pa::decode_workspace_bytes(batch, n_q, num_q_heads, d.head_dim, s_max);

  std::memset(a, 0, sizeof(*a));
  a->layout = PA_PAGED;
  a->dtype = d.dtype;
  a->H_kv = d.num_kv_heads;
  a->H_q = num_q_heads;
  a->D = d.head_dim;
  a->n_q = n_q;
  a->num_blocks = d.num_blocks;
  a->k = pool->k;
  a->v = pool->v;
  a->q = q;
  a->q_row_stride = q_row_stride;
  a->block_tables = block_tables;
  a->bt_stride = bt_stride;
  a->kv_lens = kv_lens;
  a->batch = batch;
  a->max_kv_len = max_kv_len;
  a->s_max = s_max;
  a->scale = scale;
  a->out = out;
  a->lse = lse;
  return PA_OK;
}

// Validation and argument pack of the right-padded lockstep decode.
pa_status padded_decode_prepare(const pa_pool* padded_pool, const void* q, int32_t num_q_heads,
                                int32_t batch, const int32_t* gap_start, const int32_t* gap_end,
                                int32_t kv_cols, float scale, float* out, float* lse,
                                pa::DecodeArgs* a, size_t* need) {
  pa_status s = check_pool(padded_pool);
  if (s != PA_OK) return s;
  const pa_pool_desc& d = padded_pool->desc;
  if (d.layout != PA_PADDED) return PA_ERR_SHAPE;
  if (q == nullptr || gap_start == nullptr || gap_end == nullptr || out == nullptr)
    return PA_ERR_NULL;
  if (batch < 0 || batch > d.batch_cap || batch > pa::kMaxGridYZ || kv_cols < 0 ||
      kv_cols > d.seq_cap)
    return PA_ERR_SHAPE;
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0) return PA_ERR_SHAPE;
  const int G = num_q_heads / d.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  const long long row_stride = (long long)num_q_heads * d.head_dim;
  if (!q_aligned(q, row_stride, d.dtype)) return PA_ERR_SHAPE;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;

  const int s_max = pa::num_splits(kv_cols, pa::chunk_tokens(d.head_dim));
  if (s_max > pa::kMaxGridYZ) return PA_ERR_SHAPE;
  *need = pa::decode_workspace_bytes(batch, 1, num_q_heads, d.head_dim, s_max);

  std::memset(a, 0, sizeof(*a));
  a->layout = PA_PADDED;
  a->dtype = d.dtype;
  a->H_kv = d.num_kv_heads;
  a->H_q = num_q_heads;
  a->D = d.head_dim;
  a->n_q = 1;
  a->seq_cap = d.seq_cap;
  a->k = padded_pool->k;
  a->v = padded_pool->v;
  a->q = q;
  a->q_row_stride = row_stride;
  a->gap_start = gap_start;
  a->gap_end = gap_end;
  a->kv_cols = kv_cols;
  a->batch = batch;
  a->max_kv_len = kv_cols;
  a->s_max = s_max;
  a->scale = scale;
  a->out = out;
  a->lse = lse;
  return PA_OK;
}

// The workspace query, the capacity check and the launches of a prepared decode (the split
// kernel or the multi-query kernel, then the log-sum-exp merge when rows can split).
pa_status run_decode(pa::DecodeArgs& a, size_t need, void* workspace, size_t workspace_bytes,
                     size_t* workspace_needed, hipStream_t stream) {
  if (workspace_needed != nullptr) {
    *workspace_needed = need;
    return PA_OK;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_CAPACITY;
  // counters are updated by device-scope atomics and partials stored as aligned vectors
  if (need > 0 && ((uintptr_t)workspace % 256) != 0) return PA_ERR_CAPACITY;
  if (a.batch == 0) return PA_OK;
  if (need > 0)
    pa::carve_workspace(workspace, a.batch, a.n_q, a.H_q, a.D, a.s_max,
                        pa::merge_count_bytes(a.batch, a.H_q), &a.counter, &a.part_o,
                        &a.part_lse, &a.merge_counts);
  bool merged = false;
  hipError_t e = a.n_q == 1 ? pa::launch_decode_vector(a, stream, &merged)
                            : pa::launch_decode_mq(a, stream);
  if (e == hipSuccess && a.s_max > 1 && !merged) e = pa::launch_lse_reduce(a, stream);
  return map_hip(e);
}

}  // namespace

extern "C" pa_status pa_decode_attention(const pa_pool* pool, const void* q, int64_t q_row_stride,
                                         int32_t n_q, int32_t num_q_heads,
                                         const int32_t* block_tables, int32_t bt_stride,
                                         const int32_t* kv_lens, int32_t batch,
                                         int32_t max_kv_len, float scale, void* workspace,
                                         size_t workspace_bytes, size_t* workspace_needed,
                                         float* out, float* lse, hipStream_t stream) {
  pa::DecodeArgs a;
  size_t need = 0;
  const pa_status s = paged_decode_prepare(pool, q, q_row_stride, n_q, num_q_heads, block_tables,
                                           bt_stride, kv_lens, batch, max_kv_len, scale, out, lse,
                                           &a, &need);
  if (s != PA_OK) return s;
  return run_decode(a, need, workspace, workspace_bytes, workspace_needed, stream);
}

// ---- the allocation-free decode -----------------------------------------------------------------
// pa_decode_attention_noalloc runs the split paths on the library's own scratch instead of a
// caller's workspace. `scratch` is a file-scope device array: the runtime gives every device the
// library runs on its own copy, which lives until the process ends. In host code its name is only a
// stand-in for the symbol, never a device address: the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch[device]. Layout: the
// work counters (256 bytes), a fixed reservation for the finished-split counts
// (the same offsets for every batch, so calls of any size follow one another with no clearing),
// then the partials. The counters must be zero before a call, and every completed call leaves them
// at zero; they are cleared by a fill kernel on a device's first call and after a failed launch.
namespace {

constexpr size_t kNoallocCountBytes = (size_t)PA_NOALLOC_MAX_ROW_HEADS * sizeof(int);
static_assert(kNoallocCountBytes % 256 == 0, "count reservation keeps the partials aligned");
static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

// zero n 16-byte words (the counter region of the scratch)
__global__ void clear_words_kernel(uint4* p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
  void* ptr = nullptr;  // device address of this device's `scratch`
  bool dirty = true;    // the counters may be nonzero: clear them before the next launch
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

// This device's scratch, set up on first use; clears the counters (on `stream`, ahead of the
// caller's launch) when they may be nonzero. Under stream capture the clear is recorded into the
// graph and the slot stays marked, so the next eager call clears again.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr, int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[dev];
  if (slot.ptr == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p % 256) != 0) return hipErrorInvalidSymbol;
    slot.ptr = p;
    slot.dirty = true;
  }
  if (slot.dirty) {
    const int words = (int)((pa::kCounterBytes + kNoallocCountBytes) / 16);
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint4*>(slot.ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
      slot.dirty = false;
  }
  *ptr = slot.ptr;
  *dev_out = dev;
  return hipSuccess;
}

void noalloc_mark_dirty(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch[dev].dirty = true;
}

}  // namespace

extern "C" pa_status pa_decode_attention_noalloc(const pa_pool* pool, const void* q,
                                                 int64_t q_row_stride, int32_t n_q,
                                                 int32_t num_q_heads, const int32_t* block_tables,
                                                 int32_t bt_stride, const int32_t* kv_lens,
                                                 int32_t batch, int32_t max_kv_len, float scale,
                                                 float* out, float* lse, hipStream_t stream) {
  pa::DecodeArgs a;
  size_t need = 0;
  const pa_status s = paged_decode_prepare(pool, q, q_row_stride, n_q, num_q_heads, block_tables,
                                           bt_stride, kv_lens, batch, max_kv_len, scale, out, lse,
                                           &a, &need);
  if (s != PA_OK) return s;
  size_t need_s = 0;
  if (need > 0) {
    if (pa::merge_count_bytes(a.batch, a.H_q) > kNoallocCountBytes) return PA_ERR_CAPACITY;
    need_s = pa::decode_workspace_bytes(a.batch, a.n_q, a.H_q, a.D, a.s_max, kNoallocCountBytes);
    if (need_s > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_CAPACITY;
  }
  if (a.batch == 0) return PA_OK;
  int dev = -1;
  if (need_s > 0) {
    void* ws = nullptr;
    if (noalloc_scratch(stream, &ws, &dev) != hipSuccess) return PA_ERR_HIP;
    pa::carve_workspace(ws, a.batch, a.n_q, a.H_q, a.D, a.s_max, kNoallocCountBytes, &a.counter,
                        &a.part_o, &a.part_lse, &a.merge_counts);
  }
  bool merged = false;
  hipError_t e = a.n_q == 1 ? pa::launch_decode_vector(a, stream, &merged)
                            : pa::launch_decode_mq(a, stream);
  if (e == hipSuccess && a.s_max > 1 && !merged) e = pa::launch_lse_reduce(a, stream);
  if (e != hipSuccess && dev >= 0) noalloc_mark_dirty(dev);
  return map_hip(e);
}

extern "C" pa_status pa_tokenize_kv(const pa_pool* pool, const float* neuron_table,
                                    int32_t neuron_rows, const float* time_table,
                                    int32_t time_rows, const float* value_table,
                                    int32_t value_rows, int32_t model_dim,
                                    const void* w_k_packed, const void* w_v_packed,
                                    const int32_t* offsets,
                                    const int32_t* neuron_ids, const int32_t* time_bins,
                                    const int32_t* value_ids, int32_t num_events,
                                    const int32_t* block_tables, int32_t bt_stride,
                                    int32_t batch, int32_t max_events, hipStream_t stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  const pa_pool_desc& d = pool->desc;
  if (d.layout != PA_PAGED) return PA_ERR_SHAPE;
  if (neuron_table == nullptr || time_table == nullptr || value_table == nullptr ||
      w_k_packed == nullptr || w_v_packed == nullptr || offsets == nullptr ||
      neuron_ids == nullptr || time_bins == nullptr || value_ids == nullptr ||
      block_tables == nullptr)
    return PA_ERR_NULL;
  if (d.dtype != PA_BF16) return PA_ERR_UNSUPPORTED;  // matrix-core path: bf16 pool
  if (model_dim < 32 || model_dim % 32 != 0 || model_dim > pa::tokenize_max_model_dim())
    return PA_ERR_UNSUPPORTED;
  if (neuron_rows < 1 || time_rows < 1 || value_rows < 1) return PA_ERR_SHAPE;
  if (batch < 0 || batch > pa::kMaxGridYZ || bt_stride < 1 || max_events < 0 || num_events < 0)
    return PA_ERR_SHAPE;
  if ((int64_t)max_events > (int64_t)bt_stride * pa::kBlock) return PA_ERR_SHAPE;
  const uintptr_t align = (uintptr_t)neuron_table | (uintptr_t)time_table |
                          (uintptr_t)value_table | (uintptr_t)w_k_packed |
                          (uintptr_t)w_v_packed;
  if (align % 16 != 0) return PA_ERR_SHAPE;  // 16-byte vector loads
  if (batch == 0 || max_events == 0 || num_events == 0) return PA_OK;

  pa::TokenizeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.H = d.num_kv_heads;
  a.dh = d.head_dim;
  a.model_dim = model_dim;
  a.num_blocks = d.num_blocks;
  a.k = pool->k;
  a.v = pool->v;
  a.n_emb = neuron_table;
  a.t_emb = time_table;
  a.v_emb = value_table;
  a.neuron_rows = neuron_rows;
  a.time_rows = time_rows;
  a.value_rows = value_rows;
  a.w_k = w_k_packed;
  a.w_v = w_v_packed;
  a.offsets = offsets;
  a.neuron_ids = neuron_ids;
  a.time_bins = time_bins;
  a.value_ids = value_ids;
  a.num_events = num_events;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.batch = batch;
  a.max_events = max_events;
  return map_hip(pa::launch_tokenize(a, stream));
}

extern "C" pa_status pa_pack_projection(const void* w, int32_t out_features, int32_t in_features,
                                        void* packed, hipStream_t stream) {
  if (w == nullptr || packed == nullptr) return PA_ERR_NULL;
  if (out_features < 16 || out_features % 16 != 0 || in_features < 32 || in_features % 32 != 0)
    return PA_ERR_SHAPE;
  if (((uintptr_t)w | (uintptr_t)packed) % 16 != 0) return PA_ERR_SHAPE;
  const uintptr_t bytes = (uintptr_t)out_features * (uintptr_t)in_features * 2;
  const uintptr_t wa = (uintptr_t)w, pb = (uintptr_t)packed;
  if (wa < pb + bytes && pb < wa + bytes) return PA_ERR_SHAPE;  // overlapping buffers
  return map_hip(pa::launch_pack_projection(w, packed, out_features, in_features, stream));
}

extern "C" pa_status pa_advance_lockstep(int32_t* positions, int32_t* kv_lens, int32_t* dest,
                                         int32_t batch, hipStream_t stream) {
  if (positions == nullptr) return PA_ERR_NULL;
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  return map_hip(pa::launch_advance(positions, kv_lens, dest, batch, stream));
}

extern "C" pa_status pa_decode_attention_block_sparse(
    const pa_pool* pool, const void* q, int64_t q_row_stride, int32_t n_q, int32_t num_q_heads,
    const int32_t* block_tables, int32_t bt_stride, const int32_t* kv_lens, int32_t batch,
    int32_t max_kv_len, float scale, const uint8_t* block_mask, int32_t mask_kv_blocks,
    float* out, float* lse, hipStream_t stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  const pa_pool_desc& d = pool->desc;
  if (d.layout != PA_PAGED) return PA_ERR_SHAPE;
  if (q == nullptr || block_tables == nullptr || kv_lens == nullptr || out == nullptr ||
      block_mask == nullptr)
    return PA_ERR_NULL;
  if (batch < 0 || batch > pa::kMaxGridYZ || n_q < 1 || bt_stride < 1 || max_kv_len < 0 ||
      q_row_stride < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_kv_len > (int64_t)bt_stride * pa::kBlock) return PA_ERR_SHAPE;
  const int64_t kv_blocks = ((int64_t)max_kv_len + pa::kBlock - 1) / pa::kBlock;
  if (mask_kv_blocks < 1 || (int64_t)mask_kv_blocks < kv_blocks) return PA_ERR_SHAPE;
  if (d.dtype != PA_BF16) return PA_ERR_UNSUPPORTED;  // matrix-core path: bf16 only
  if (!q_aligned(q, q_row_stride, d.dtype)) return PA_ERR_SHAPE;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;

  pa::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.layout = PA_PAGED;
  a.dtype = d.dtype;
  a.H_kv = d.num_kv_heads;
  a.H_q = num_q_heads;
  a.D = d.head_dim;
  a.n_q = n_q;
  a.num_blocks = d.num_blocks;
  a.k = pool->k;
  a.v = pool->v;
  a.q = q;
  a.q_row_stride = q_row_stride;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.kv_lens = kv_lens;
  a.batch = batch;
  a.max_kv_len = max_kv_len;
  a.s_max = 1;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.block_mask = block_mask;
  a.mask_kv_blocks = mask_kv_blocks;
  return map_hip(pa::launch_decode_mq(a, stream));
}

extern "C" pa_status pa_decode_attention_padded(const pa_pool* padded_pool, const void* q,
                                                int32_t num_q_heads, int32_t batch,
                                                const int32_t* gap_start, const int32_t* gap_end,
                                                int32_t kv_cols, float scale, void* workspace,
                                                size_t workspace_bytes, size_t* workspace_needed,
                                                float* out, float* lse, hipStream_t stream) {
  pa::DecodeArgs a;
  size_t need = 0;
  const pa_status s = padded_decode_prepare(padded_pool, q, num_q_heads, batch, gap_start,
                                            gap_end, kv_cols, scale, out, lse, &a, &need);
  if (s != PA_OK) return s;
  return run_decode(a, need, workspace, workspace_bytes, workspace_needed, stream);
}

namespace {

// The append half of the fused calls: checks, and the fields of the decode's argument pack.
pa_status fused_prepare(const pa_pool* pool, const int32_t* positions, const int32_t* dest,
                        const void* k_new, const void* v_new, const void* q, void* q_out,
                        pa::DecodeArgs* a) {
  const pa_pool_desc& d = pool->desc;
  if (positions == nullptr || k_new == nullptr || v_new == nullptr) return PA_ERR_NULL;
  const bool rope = d.rope_max_pos > 0;
  if (rope && q_out == nullptr) return PA_ERR_NULL;
  const long long q_stride = (long long)a->H_q * d.head_dim;
  const long long kv_stride = (long long)d.num_kv_heads * d.head_dim;
  if (!q_aligned(k_new, kv_stride, d.dtype) || !q_aligned(v_new, kv_stride, d.dtype))
    return PA_ERR_SHAPE;
  if (q_out != nullptr) {
    if (!q_aligned(q_out, q_stride, d.dtype)) return PA_ERR_SHAPE;
    // every workgroup reads q while split 0 writes q_out: they must not overlap
    const uintptr_t bytes = (uintptr_t)a->batch * (uintptr_t)q_stride * elem_size(d.dtype);
    const uintptr_t x = (uintptr_t)q, y = (uintptr_t)q_out;
    if (bytes > 0 && (x < y ? y - x : x - y) < bytes) return PA_ERR_SHAPE;
  }
  a->positions = positions;
  a->dest = dest;
  a->k_new = k_new;
  a->v_new = v_new;
  a->q_out = q_out;
  a->cos = rope ? pool->rope_cos : nullptr;
  a->sin = rope ? pool->rope_sin : nullptr;
  a->rope_max_pos = d.rope_max_pos;
  return PA_OK;
}

// One launch of the decode kernel that also appends, then the merge.
pa_status run_append_decode(pa::DecodeArgs& a, size_t need, void* workspace,
                            size_t workspace_bytes, size_t* workspace_needed,
                            hipStream_t stream) {
  if (workspace_needed != nullptr) {
    *workspace_needed = need;
    return PA_OK;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_CAPACITY;
  // counters are updated by device-scope atomics and partials stored as aligned vectors
  if (need > 0 && ((uintptr_t)workspace % 256) != 0) return PA_ERR_CAPACITY;
  if (a.batch == 0) return PA_OK;
  if (need > 0)
    pa::carve_workspace(workspace, a.batch, 1, a.H_q, a.D, a.s_max,
                        pa::merge_count_bytes(a.batch, a.H_q), &a.counter, &a.part_o,
                        &a.part_lse, &a.merge_counts);
  bool merged = false;
  hipError_t e = pa::launch_decode_vector(a, stream, &merged);
  if (e == hipSuccess && a.s_max > 1 && !merged) e = pa::launch_lse_reduce(a, stream);
  return map_hip(e);
}

}  // namespace

extern "C" pa_status pa_append_decode_attention(
    const pa_pool* pool, const int32_t* block_tables, int32_t bt_stride,
    const int32_t* positions, const int32_t* dest, const void* k_new, const void* v_new,
    const void* q, void* q_out, int32_t num_q_heads, const int32_t* kv_lens, int32_t batch,
    int32_t max_kv_len, float scale, void* workspace, size_t workspace_bytes,
    size_t* workspace_needed, float* out, float* lse, hipStream_t stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  pa::DecodeArgs a;
  size_t need = 0;
  s = paged_decode_prepare(pool, q, (int64_t)num_q_heads * pool->desc.head_dim, 1, num_q_heads,
                           block_tables, bt_stride, kv_lens, batch, max_kv_len, scale, out, lse,
                           &a, &need);
  if (s != PA_OK) return s;
  s = fused_prepare(pool, positions, dest, k_new, v_new, q, q_out, &a);
  if (s != PA_OK) return s;
  return run_append_decode(a, need, workspace, workspace_bytes, workspace_needed, stream);
}

extern "C" pa_status pa_lockstep_decode_step(
    const pa_pool* pool, const int32_t* block_tables, int32_t bt_stride, const int32_t* positions,
    int32_t* positions_out, const void* k_new, const void* v_new, const void* q, void* q_out,
    int32_t num_q_heads, int32_t batch, int32_t max_kv_len, float scale, void* workspace,
    size_t workspace_bytes, size_t* workspace_needed, float* out, float* lse,
    hipStream_t stream) {
  pa_status s = check_pool(pool);
  if (s != PA_OK) return s;
  if (positions == nullptr || positions_out == nullptr) return PA_ERR_NULL;
  // the step reads positions while one workgroup per row writes positions_out
  const uintptr_t pb = (uintptr_t)positions, po = (uintptr_t)positions_out;
  const uintptr_t pn = (uintptr_t)(batch > 0 ? batch : 0) * sizeof(int32_t);
  if (pn > 0 && pb < po + pn && po < pb + pn) return PA_ERR_SHAPE;
  pa::DecodeArgs a;
  size_t need = 0;
  // kv_lens are taken from the positions: the pointer stands in for the decode's own null check
  s = paged_decode_prepare(pool, q, (int64_t)num_q_heads * pool->desc.head_dim, 1, num_q_heads,
                           block_tables, bt_stride, positions, batch, max_kv_len, scale, out, lse,
                           &a, &need);
  if (s != PA_OK) return s;
  s = fused_prepare(pool, positions, nullptr, k_new, v_new, q, q_out, &a);
  if (s != PA_OK) return s;
  a.kv_lens = nullptr;
  a.kv_from_positions = 1;
  a.positions_out = positions_out;
  return run_append_decode(a, need, workspace, workspace_bytes, workspace_needed, stream);
}

extern "C" pa_status pa_append_decode_attention_padded(
    const pa_pool* padded_pool, const int32_t* positions, const int32_t* dest, const void* k_new,
    const void* v_new, const void* q, void* q_out, int32_t num_q_heads,
    const int32_t* gap_start, const int32_t* gap_end, int32_t kv_cols, int32_t batch,
    float scale, void* workspace, size_t workspace_bytes, size_t* workspace_needed, float* out,
    float* lse, hipStream_t stream) {
  pa::DecodeArgs a;
  size_t need = 0;
  pa_status s = padded_decode_prepare(padded_pool, q, num_q_heads, batch, gap_start, gap_end,
                                      kv_cols, scale, out, lse, &a, &need);
  if (s != PA_OK) return s;
  s = fused_prepare(padded_pool, positions, dest, k_new, v_new, q, q_out, &a);
  if (s != PA_OK) return s;
  return run_append_decode(a, need, workspace, workspace_bytes, workspace_needed, stream);
}

extern "C" pa_status pa_lse_merge(const float* out_parts, const float* lse_parts, int32_t num_parts,
                                  int64_t n, int32_t head_dim, float* out, float* lse,
                                  hipStream_t stream) {
  if (out_parts == nullptr || lse_parts == nullptr || out == nullptr) return PA_ERR_NULL;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_parts < 1 || num_parts > 65535 || n < 0 || n > ((int64_t)1 << 34)) return PA_ERR_SHAPE;
  // the outputs must not overlap the parts (every wave reads all parts of its pair)
  const uintptr_t pb = (uintptr_t)out_parts, pe = pb + (uintptr_t)num_parts * n * head_dim * 4;
  const uintptr_t ob = (uintptr_t)out, oe = ob + (uintptr_t)n * head_dim * 4;
  if (n > 0 && ob < pe && pb < oe) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  pa::LseMergeArgs a;
  a.out_parts = out_parts;
  a.lse_parts = lse_parts;
  a.num_parts = num_parts;
  a.n = n;
  a.D = head_dim;
  a.out = out;
  a.lse = lse;
  return map_hip(pa::launch_lse_merge(a, stream));
}
