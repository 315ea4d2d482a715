// append_kv for gfx950: write each row's new key (rotated at its own position) and value into the
// pool, and optionally rotate the queries at the same positions.
//
// helexa PR #121, commit "slice 1": cos/sin are gathered at arbitrary per-row positions and applied
// rotate-half (element i pairs with i + D/2); keys are stored post-RoPE, so where a key sits (its
// slot or padded column) never changes its scores. NeuroGrid releases, v0.7.0 "Paged KV Cache": the
// slot is found through the row's block table.
//
// One thread per (row, head, i < D/2) handles the pair (i, i + D/2). The rotation is done in fp32
// with every product and sum rounded on its own (contraction into fused multiply-adds is switched
// off), and the result is rounded to the pool dtype by the hardware fp32 -> bf16 conversion (round
// to nearest even), so the stored bits do not depend on the launch geometry.
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

// Raw storage bits of T: copies move bits, never values (no NaN canonicalisation).
template <typename T>
using Bits = typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type;

template <typename T>
__device__ __forceinline__ void copy_pair(const T* src, T* dst, int i, int half) {
  const Bits<T>* s = reinterpret_cast<const Bits<T>*>(src);
  Bits<T>* d = reinterpret_cast<Bits<T>*>(dst);
  d[i] = s[i];
  d[i + half] = s[i + half];
}

// r_lo = x_lo*c - x_hi*s ; r_hi = x_hi*c + x_lo*s, each operation rounded separately.
__device__ __forceinline__ void rotate_pair(float x_lo, float x_hi, float c, float s, float* r_lo,
                                            float* r_hi) {
#pragma clang fp contract(off)
  const float a = x_lo * c;
  const float b = x_hi * s;
  const float d = x_hi * c;
  const float e = x_lo * s;
  *r_lo = a - b;
  *r_hi = d + e;
}

// Grid (ceil(heads * D/2 / 256), batch): blockIdx.y is the row, so its position, destination and
// block-table entry are workgroup-uniform loads issued at once; the index inside the row needs only
// shifts (D/2 is a power of two). The D/2 lanes of one head are consecutive and aligned inside a
// wave, which is what the per-head RMSNorm (NORM) reduces over: the sum of squares of the
// rotate-half pairs, then a butterfly with lane strides 1, 2, 4, ... -- fp32 addition commutes,
// so every lane ends with the same sum, formed as a pairwise tree of neighbours.
template <typename T, bool NORM>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a, int log2_half) {
#pragma clang fp contract(off)
  const int half = 1 << log2_half;
  const int heads = 2 * a.H_kv + (a.q_in != nullptr ? a.H_q : 0);
  const int idx = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int b = (int)blockIdx.y;
  const bool live = idx < heads * half;
  const int i = idx & (half - 1);
  const int hh = live ? idx >> log2_half : 0;
  const bool is_q = hh >= 2 * a.H_kv;
  const bool is_v = !is_q && hh >= a.H_kv;
  const int h = is_q ? hh - 2 * a.H_kv : (is_v ? hh - a.H_kv : hh);

  const bool rope = a.cos != nullptr;
  int pos = a.positions[b];
  if (rope) pos = clampi(pos, 0, a.rope_max_pos - 1);

  const T* src = is_q ? reinterpret_cast<const T*>(a.q_in) + ((size_t)b * a.H_q + h) * a.D
                      : reinterpret_cast<const T*>(is_v ? a.v_new : a.k_new) +
                            ((size_t)b * a.H_kv + h) * a.D;
  float x_lo = 0.f, x_hi = 0.f;
  if (live && !is_v) {
    x_lo = to_f32(src[i]);
    x_hi = to_f32(src[i + half]);
  }
  if constexpr (NORM) {
    // every lane takes part (no lane has returned yet); a head's lanes never mix with another's
    float ss = x_lo * x_lo + x_hi * x_hi;
    for (int m = 1; m < half; m <<= 1) ss = ss + __shfl_xor(ss, m);
    const float ms = ss / (float)a.D;
    const float r = 1.0f / sqrtf(ms + a.norm_eps);
    if (live && !is_v) {
      const float* w = is_q ? a.q_norm_w : a.k_norm_w;
      x_lo = (x_lo * r) * w[i];
      x_hi = (x_hi * r) * w[i + half];
    }
  }
  if (!live) return;

  // rotated (and/or normalised) values, or the raw bits when neither applies
  auto store_pair = [&](T* dst) {
    if (rope) {
      float r_lo, r_hi;
      rotate_pair(x_lo, x_hi, a.cos[(size_t)pos * half + i], a.sin[(size_t)pos * half + i], &r_lo,
                  &r_hi);
      dst[i] = from_f32<T>(r_lo);
      dst[i + half] = from_f32<T>(r_hi);
    } else if (NORM) {
      dst[i] = from_f32<T>(x_lo);
      dst[i + half] = from_f32<T>(x_hi);
    } else {
      copy_pair(src, dst, i, half);
    }
  };

  if (is_q) {  // query head: into q_out
    store_pair(reinterpret_cast<T*>(a.q_out) + ((size_t)b * a.H_q + h) * a.D);
    return;
  }
  int t = a.dest != nullptr ? a.dest[b] : a.positions[b];
  size_t slot_base;  // element offset of [.., h, slot/column, 0]
  if (a.layout == PA_PAGED) {
    t = clampi(t, 0, a.bt_stride * kBlock - 1);
    int blk = a.block_tables[(size_t)b * a.bt_stride + t / kBlock];
    blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
    slot_base = (((size_t)blk * a.H_kv + h) * kBlock + (t % kBlock)) * a.D;
  } else {
    t = clampi(t, 0, a.seq_cap - 1);
    slot_base = (((size_t)b * a.H_kv + h) * a.seq_cap + t) * a.D;
  }
  if (is_v) {
    copy_pair(src, reinterpret_cast<T*>(a.v) + slot_base, i, half);
    return;
  }
  store_pair(reinterpret_cast<T*>(a.k) + slot_base);
}

// Advance a lockstep batch by one token: position += 1, kv_len = position + 1, dest += 1
// (unsigned arithmetic: a position at the int32 limit wraps instead of overflowing).
__global__ __launch_bounds__(256) void advance_kernel(int32_t* positions, int32_t* kv_lens,
                                                      int32_t* dest, int batch) {
  const int b = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (b >= batch) return;
  const uint32_t p = (uint32_t)positions[b] + 1u;
  positions[b] = (int32_t)p;
  if (kv_lens != nullptr) kv_lens[b] = (int32_t)(p + 1u);
  if (dest != nullptr) dest[b] = (int32_t)((uint32_t)dest[b] + 1u);
}

}  // namespace

hipError_t launch_advance(int32_t* positions, int32_t* kv_lens, int32_t* dest, int batch,
                          hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream,
                     positions, kv_lens, dest, batch);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int heads = 2 * a.H_kv + (a.q_in != nullptr ? a.H_q : 0);
  const int half = a.D / 2;
  if (a.batch <= 0 || heads * half == 0) return hipSuccess;
  int log2_half = 0;
  while ((1 << log2_half) < half) ++log2_half;
  if ((1 << log2_half) != half) return hipErrorInvalidValue;  // head_dim is 32, 64 or 128
  const dim3 grid((unsigned)((heads * half + 255) / 256), (unsigned)a.batch);
  const bool norm = a.k_norm_w != nullptr;
  if (a.dtype == PA_F32) {
    if (norm)
      hipLaunchKernelGGL((append_kernel<float, true>), grid, dim3(256), 0, stream, a, log2_half);
    else
      hipLaunchKernelGGL((append_kernel<float, false>), grid, dim3(256), 0, stream, a, log2_half);
  } else {
    if (norm)
      hipLaunchKernelGGL((append_kernel<__bf16, true>), grid, dim3(256), 0, stream, a, log2_half);
    else
      hipLaunchKernelGGL((append_kernel<__bf16, false>), grid, dim3(256), 0, stream, a,
                         log2_half);
  }
  return hipGetLastError();
}

}  // namespace pa
