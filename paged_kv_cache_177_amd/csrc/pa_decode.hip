// Single-query decode attention over the paged (or right-padded) K/V cache, for gfx950.
//
// What it computes: for every row b and query head h, softmax(scale * q_h . K^T) V over the row's
// valid tokens, reading K/V through the row's block table (NeuroGrid releases, v0.7.0 "Paged KV
// Cache": block-table paged attention with GQA) with an online softmax that never materialises the
// scores (v0.6.0 "Flash Decode Attention Kernel"; cortex-engine write-up, kernels section: running
// max, running sum and output statistics; a fully masked row gives zeros). The padded form skips
// each row's padding gap [gap_start, gap_end) (helexa PR #121, commit "slice 1":
// batch_decode_mask over one gap per row).
//
// Mapping (one workgroup = 4 waves per (KV head g, row b, split s)):
//   * A row is cut into chunks of chunk_tokens(D) tokens; split s owns chunk s. The workgroup
//     covers the G = H_q / H_kv query heads of KV head g, so every K/V byte is loaded once and
//     used by all G heads straight from registers.
//   * Inside a wave, LPT = D/16 lanes share one token (16 dims each); a "step" is the 64/LPT
//     tokens one wave loads at once (exactly one 16-token block at D = 64). Steps of the chunk are
//     dealt round-robin to the 4 waves; each wave prefetches its next step's K and V (one
//     contiguous 16-byte-per-lane read per tensor) while it computes the current one.
//   * q.k: packed bf16 dot products (v_dot2_f32_bf16) accumulate in fp32, then a DPP butterfly
//     over the LPT lanes of the token. Scores are kept in log2 units (scale * log2(e) folded in)
//     so the softmax uses the hardware exp2.
//   * Online softmax per lane: each lane keeps its own running max m, sum l and accumulator for
//     the tokens it sees. m is only raised when a score exceeds it by more than 2^8 (log2 units),
//     so rescaling is rare; all weights stay <= 2^8 and the result is exact up to rounding.
//   * At the end lanes are merged with a common max: DPP inside each 16-lane row, then LDS across
//     rows and waves. One split writes out/lse; several splits write normalised partials and their
//     log-sum-exp, merged by lse_reduce_kernel.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 units
constexpr int kWaves = 4;
constexpr float kNegInf = -__builtin_inff();

// ---- cross-lane helpers (DPP) --------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i inside each 8-lane half row
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return dpp<0x120 + N>(x);
}

// Sum over the LPT consecutive lanes that share one token (result in all of them).
template <int LPT>
__device__ __forceinline__ float token_lane_sum(float x) {
  static_assert(LPT == 2 || LPT == 4 || LPT == 8, "lanes per token");
  x += dpp<kQuadXor1>(x);
  if constexpr (LPT >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (LPT >= 8) x += dpp<kRowHalfMirror>(x);
  return x;
}

// Reduce over the token streams of one 16-lane row (lanes congruent mod LPT); result in all.
template <int LPT, bool MAX>
__device__ __forceinline__ float row_stream_reduce(float x) {
  if constexpr (LPT <= 1) x = MAX ? fmaxf(x, row_ror<1>(x)) : x + row_ror<1>(x);
  if constexpr (LPT <= 2) x = MAX ? fmaxf(x, row_ror<2>(x)) : x + row_ror<2>(x);
  if constexpr (LPT <= 4) x = MAX ? fmaxf(x, row_ror<4>(x)) : x + row_ror<4>(x);
  if constexpr (LPT <= 8) x = MAX ? fmaxf(x, row_ror<8>(x)) : x + row_ror<8>(x);
  return x;
}

// Lane i <-> lane i ^ 16 (inside each 32-lane half): ds_swizzle in bit-mask mode
// (and_mask 0x1f, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ float swap_rows16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
// Lane i <-> lane i ^ 32.
__device__ __forceinline__ float swap_halves32(float x) { return __shfl_xor(x, 32); }

// Sum over all token streams of the wave (lanes congruent mod LPT); result in all lanes.
template <int LPT>
__device__ __forceinline__ float wave_stream_sum(float x) {
  x = row_stream_reduce<LPT, false>(x);
  x += swap_rows16(x);
  x += swap_halves32(x);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// ---- per-dtype register fragments (16 elements of one token per lane) ---------------------------
template <typename T>
struct Frag;

template <>
struct Frag<__bf16> {
  uint4 k[2], v[2];
  __device__ __forceinline__ void load(const __bf16* kp, const __bf16* vp) {
    const uint4* a = reinterpret_cast<const uint4*>(kp);
    const uint4* b = reinterpret_cast<const uint4*>(vp);
    k[0] = a[0];
    k[1] = a[1];
    v[0] = b[0];
    v[1] = b[1];
  }
  __device__ __forceinline__ void zero_v() { v[0] = v[1] = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void v_f32(float* o) const {
    const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = bf16_lo(w[i]);
      o[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};

template <>
struct Frag<float> {
  float4 k[4], v[4];
  __device__ __forceinline__ void load(const float* kp, const float* vp) {
    const float4* a = reinterpret_cast<const float4*>(kp);
    const float4* b = reinterpret_cast<const float4*>(vp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[i] = a[i];
      v[i] = b[i];
    }
  }
  __device__ __forceinline__ void zero_v() {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ void v_f32(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[4 * i] = v[i].x;
      o[4 * i + 1] = v[i].y;
      o[4 * i + 2] = v[i].z;
      o[4 * i + 3] = v[i].w;
    }
  }
};

// Query registers of one lane: 16 dims of each of the G heads.
template <typename T, int G>
struct QRegs;

template <int G>
struct QRegs<__bf16, G> {
  uint32_t q[G][8];
  __device__ __forceinline__ void load(const __bf16* p, int head_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4* a = reinterpret_cast<const uint4*>(p + (size_t)h * head_stride);
      uint4 x = a[0], y = a[1];
      q[h][0] = x.x; q[h][1] = x.y; q[h][2] = x.z; q[h][3] = x.w;
      q[h][4] = y.x; q[h][5] = y.y; q[h][6] = y.z; q[h][7] = y.w;
    }
  }
  __device__ __forceinline__ float dot(int h, const Frag<__bf16>& f) const {
    const uint32_t w[8] = {f.k[0].x, f.k[0].y, f.k[0].z, f.k[0].w,
                           f.k[1].x, f.k[1].y, f.k[1].z, f.k[1].w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[h][i]),
                                          __builtin_bit_cast(bf16x2_t, w[i]), a, false);
      b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[h][i + 1]),
                                          __builtin_bit_cast(bf16x2_t, w[i + 1]), b, false);
    }
    return a + b;
  }
};

template <int G>
struct QRegs<float, G> {
  float q[G][16];
  __device__ __forceinline__ void load(const float* p, int head_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4* a = reinterpret_cast<const float4*>(p + (size_t)h * head_stride);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 x = a[i];
        q[h][4 * i] = x.x; q[h][4 * i + 1] = x.y; q[h][4 * i + 2] = x.z; q[h][4 * i + 3] = x.w;
      }
    }
  }
  __device__ __forceinline__ float dot(int h, const Frag<float>& f) const {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a = fmaf(q[h][4 * i], f.k[i].x, a);
      b = fmaf(q[h][4 * i + 1], f.k[i].y, b);
      a = fmaf(q[h][4 * i + 2], f.k[i].z, a);
      b = fmaf(q[h][4 * i + 3], f.k[i].w, b);
    }
    return a + b;
  }
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---- the kernel ------------------------------------------------------------------------------
template <typename T, int D, int G, bool PADDED>
__global__ __launch_bounds__(256) void decode_vector_kernel(const DecodeArgs a) {
  constexpr int LPT = D / 16;    // lanes per token
  constexpr int TPS = 64 / LPT;  // tokens per wave step
  const int g = blockIdx.x;
  const int row = blockIdx.y;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tl = lane / LPT;
  const int c = lane % LPT;

  // valid tokens of the row
  int n, gap_s = 0, gap_shift = 0;
  if constexpr (PADDED) {
    const int cols = a.kv_cols;
    gap_s = clampi(a.gap_start[row], 0, cols);
    const int gap_e = clampi(a.gap_end[row], gap_s, cols);
    gap_shift = gap_e - gap_s;
    n = cols - gap_shift;
  } else {
    n = clampi(a.kv_lens[row], 0, a.max_kv_len);
  }
  const int chunk = chunk_tokens(D);
  const int ns = num_splits(n, chunk);
  if (split >= ns) return;
  const int tok0 = split * chunk;
  const int ntok = n - tok0 < chunk ? n - tok0 : chunk;  // >= 0
  const int nsteps = (ntok + TPS - 1) / TPS;

  const T* __restrict__ kbase = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ vbase = reinterpret_cast<const T*>(a.v);

  // block ids of this chunk: lane i holds logical block (tok0/16 + i)
  int ids = 0;
  size_t head_base = 0;
  if constexpr (!PADDED) {
    const int nblk = (ntok + kBlock - 1) / kBlock;
    if (lane < nblk) {
      int v = a.block_tables[(size_t)row * a.bt_stride + (tok0 >> 4) + lane];
      ids = (unsigned)v < (unsigned)a.num_blocks ? v : 0;
    }
  } else {
    head_base = ((size_t)row * a.H_kv + g) * (size_t)a.seq_cap * D;
  }

  // queries of the G heads of group g, this lane's 16 dims
  QRegs<T, G> q;
  q.load(reinterpret_cast<const T*>(a.q) + (size_t)row * a.q_row_stride + (size_t)g * G * D + c * 16,
         D);
  const float qk_scale = a.scale * kLog2e;

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  // element offset of this lane's 16 dims of token t (relative to the chunk start)
  auto offset_of = [&](int step, int t) -> size_t {
    if constexpr (PADDED) {
      int tv = tok0 + t;
      int col = tv < gap_s ? tv : tv + gap_shift;
      col = col < a.kv_cols ? col : a.kv_cols - 1;
      return head_base + (size_t)col * D + c * 16;
    } else {
      int pb;
      if constexpr (TPS <= kBlock) {
        pb = __builtin_amdgcn_readlane(ids, (step * TPS) >> 4);
      } else {
        pb = __shfl(ids, t >> 4);
      }
      return (((size_t)pb * a.H_kv + g) * kBlock + (t & (kBlock - 1))) * D + c * 16;
    }
  };

  const int my_steps = wave < nsteps ? (nsteps - wave + kWaves - 1) / kWaves : 0;
  Frag<T> cur;
  if (my_steps > 0) {
    const int t = wave * TPS + tl;
    const size_t off = offset_of(wave, t);
    cur.load(kbase + off, vbase + off);
  }
  for (int i = 0; i < my_steps; ++i) {
    const int step = wave + i * kWaves;
    Frag<T> nxt;
    if (i + 1 < my_steps) {
      const int s2 = step + kWaves;
      const size_t off = offset_of(s2, s2 * TPS + tl);
      nxt.load(kbase + off, vbase + off);
    }
    const int t = step * TPS + tl;
    const bool tail = (step + 1) * TPS > ntok;  // wave-uniform
    const bool valid = t < ntok;
    if (tail && !valid) cur.zero_v();

    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = token_lane_sum<LPT>(q.dot(h, cur)) * qk_scale;
    if (tail) {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = valid ? s[h] : kNegInf;
    }
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= s[h] > m[h] + kRescale;
    if (need) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = s[h] > m[h] + kRescale ? s[h] : m[h];
        const float al = exp2_fast(m[h] - mn);
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] *= al;
        m[h] = mn;
      }
    }
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = exp2_fast(s[h] - m[h]);
      if (tail) p[h] = valid ? p[h] : 0.f;
      l[h] += p[h];
    }
    float vf[16];
    cur.v_f32(vf);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(p[h], vf[e], acc[h][e]);
    cur = nxt;
  }

  // ---- merge the lanes' streams to one (m, l, acc) per wave: DPP inside each 16-lane row, then
  // a swizzle across the two rows of each half-wave and a swap across the two half-waves ----------
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mr = row_stream_reduce<LPT, true>(m[h]);
    mr = fmaxf(mr, swap_rows16(mr));
    mr = fmaxf(mr, swap_halves32(mr));
    const float f = (m[h] == kNegInf) ? 0.f : exp2_fast(m[h] - mr);
    l[h] = wave_stream_sum<LPT>(l[h] * f);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = wave_stream_sum<LPT>(acc[h][e] * f);
    m[h] = mr;
  }
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_acc[wave][h][c * 16 + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  const int H_q = a.H_kv * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D;
    const int d = idx % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][h];
      const float f = (mw == kNegInf) ? 0.f : exp2_fast(mw - mx);
      A = fmaf(f, s_acc[w][h][d], A);
      L = fmaf(f, s_l[w][h], L);
    }
    const float o = L > 0.f ? A / L : 0.f;
    const float lse2 = L > 0.f ? mx + __log2f(L) : kNegInf;
    const int hq = g * G + h;
    if (ns == 1) {
      a.out[((size_t)row * H_q + hq) * D + d] = o;
      if (a.lse != nullptr && d == 0) a.lse[(size_t)row * H_q + hq] = lse2 * kLn2;
    } else {
      const size_t pr = ((size_t)row * H_q + hq) * a.s_max + split;
      a.part_o[pr * D + d] = o;
      if (d == 0) a.part_lse[pr] = lse2;
    }
  }
}

// Merge the split partials of one (row, query head): out = sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - max lse), lse = max + log2(sum w_s) (returned in natural-log units).
template <bool PADDED>
__global__ __launch_bounds__(128) void lse_reduce_kernel(const DecodeArgs a) {
  const int hq = blockIdx.x;
  const int row = blockIdx.y;
  const int d = threadIdx.x;
  int n;
  if constexpr (PADDED) {
    const int gs = clampi(a.gap_start[row], 0, a.kv_cols);
    const int ge = clampi(a.gap_end[row], gs, a.kv_cols);
    n = a.kv_cols - (ge - gs);
  } else {
    n = clampi(a.kv_lens[row], 0, a.max_kv_len);
  }
  const int ns = num_splits(n, chunk_tokens(a.D));
  if (ns <= 1 || d >= a.D) return;
  const int H_q = a.H_q;
  const size_t base = ((size_t)row * H_q + hq) * a.s_max;
  float mx = kNegInf;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_lse[base + s]);
  float A = 0.f, W = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.part_lse[base + s];
    const float f = (ls == kNegInf) ? 0.f : exp2_fast(ls - mx);
    W += f;
    A = fmaf(f, a.part_o[(base + s) * a.D + d], A);
  }
  a.out[((size_t)row * H_q + hq) * a.D + d] = W > 0.f ? A / W : 0.f;
  if (a.lse != nullptr && d == 0)
    a.lse[(size_t)row * H_q + hq] = W > 0.f ? (mx + __log2f(W)) * kLn2 : kNegInf;
}

template <typename T, int D, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.H_kv, a.batch, a.s_max);
  if (a.layout == PA_PADDED)
    hipLaunchKernelGGL((decode_vector_kernel<T, D, G, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_vector_kernel<T, D, G, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_typed<T, D, 1>(a, stream);
    case 2: return launch_typed<T, D, 2>(a, stream);
    case 4: return launch_typed<T, D, 4>(a, stream);
    case 8: return launch_typed<T, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 32: return launch_d<T, 32>(a, stream);
    case 64: return launch_d<T, 64>(a, stream);
    case 128: return launch_d<T, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_vector(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == PA_F32 ? launch_t<float>(a, stream) : launch_t<__bf16>(a, stream);
}

hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.H_q * a.n_q, a.batch);
  if (a.layout == PA_PADDED)
    hipLaunchKernelGGL(lse_reduce_kernel<true>, grid, dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL(lse_reduce_kernel<false>, grid, dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
