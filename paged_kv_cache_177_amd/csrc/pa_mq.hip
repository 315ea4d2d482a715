// Multi-query paged attention on the gfx950 matrix cores: many queries per row attend to the row's
// ragged keys, read through its block table from the same 16-token block pool (cortex-engine
// write-up, kernels section: latent queries cross-attend to a variable number of spike tokens, with
// a FlashAttention-2 style online softmax; a fully masked row gives zeros).
//
// Query "rows" of KV head g are the (query i, head h) pairs with h in g's group: r = i * G + (h - gG).
// One workgroup (4 waves) takes 16 query rows of one (row b, KV head g); its waves split the row's
// 16-token key blocks round-robin and merge through LDS at the end. Per block, per wave:
//   S^T[16 keys][16 q] = K[16 keys][D] . Q^T[D][16 q]   v_mfma_f32_16x16x32_bf16, D/32 steps
//       K is the A operand straight from the block (lane: key l%16, 8 dims), Q^T the B operand
//       (lane: query l%16, 8 dims); the result puts query l%16 in lane l, keys 4(l/16)..+3.
//   online softmax per query: lane-local, plus two cross-lane steps for the block maximum;
//   O^T[D][16 q] += V^T[D][16 keys] . P^T[16 keys][16 q]   v_mfma_f32_16x16x16_bf16, D/16 steps
//       P^T is the B operand exactly as the first product left it (query l%16, keys 4(l/16)..);
//       V^T (lane: dim l%16, keys 4(l/16)..) is read transposed from the block staged in LDS.
//       P is split into bf16 hi + lo parts (two products), so the weights keep ~16 bits.
// Query rows therefore sit in the same lanes in S^T and O^T: rescales and the final division are
// lane-local.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 units
constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = 4;
constexpr int kTileRows = 16;

__device__ __forceinline__ float swap_rows16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float swap_halves32(float x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion)
__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_value(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

template <int D>
struct MqSmem {
  unsigned short v[kWaves][kBlock * D];  // each wave's staged V block
  float o[kWaves][D][kTileRows];
  float m[kWaves][kTileRows];
  float l[kWaves][kTileRows];
};

template <int D>
__global__ __launch_bounds__(64 * kWaves) void mq_paged_mfma_kernel(const DecodeArgs a) {
  constexpr int KC = D / 32;  // k-steps of the score product
  constexpr int NH = D / 16;  // dim tiles of the output product
  __shared__ MqSmem<D> sm;
  const int tile = blockIdx.x;
  const int g = blockIdx.y;
  const int row = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // query row inside the tile (S^T / O^T column)
  const int grp = lane >> 4;  // key group: keys 4*grp .. 4*grp+3 of a block
  const int G = a.H_q / a.H_kv;
  const int R = a.n_q * G;  // query rows of this KV head
  const int r = tile * kTileRows + col;
  const bool row_ok = r < R;
  const int qi = row_ok ? r / G : 0;
  const int qh = g * G + (row_ok ? r % G : 0);

  // Q^T fragments (B operand): query r, dims 32c + 8 grp .. +7; zero for rows past R
  bf16x8_t qf[KC];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (size_t)row * a.q_row_stride +
                       ((size_t)qi * a.H_q + qh) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row_ok) x = *reinterpret_cast<const u32x4_t*>(qp + 32 * c);
      qf[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  const int n = clampi(a.kv_lens[row], 0, a.max_kv_len);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int* bt = a.block_tables + (size_t)row * a.bt_stride;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v);
  const float qk_scale = a.scale * kLog2e;

  float m = kNegInf, l = 0.f;
  f32x4_t o[NH];
#pragma unroll
  for (int t = 0; t < NH; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K fragment (A operand): key col of the block, dims 32c + 8 grp; V: 16 contiguous bytes per lane
  // at lane * 8 elements (its transpose is read back from LDS)
  struct Frag {
    u32x4_t k[KC];
    u32x4_t v[D / 32];
  };
  auto load = [&](Frag& f, int blk) {
    int pb = bt[blk];
    pb = (unsigned)pb < (unsigned)a.num_blocks ? pb : 0;
    const size_t base = ((size_t)pb * a.H_kv + g) * (size_t)(kBlock * D);
    const __bf16* kb = kbase + base + (size_t)col * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c) f.k[c] = *reinterpret_cast<const u32x4_t*>(kb + 32 * c);
    const __bf16* vb = vbase + base + (size_t)lane * 8;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) f.v[c] = *reinterpret_cast<const u32x4_t*>(vb + 512 * c);
  };
  auto compute = [&](const Frag& f, int blk) {
    // stage V in this wave's LDS area ([16 keys][D]); the wave reads it back transposed
    u32x4_t* vs = reinterpret_cast<u32x4_t*>(sm.v[wave]);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) vs[lane + 64 * c] = f.v[c];
    __builtin_amdgcn_wave_barrier();

    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.k[c]), qf[c], s,
                                                  0, 0, 0);
    const int key0 = blk * kBlock + 4 * grp;
    bool valid[4];
    float bm = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      valid[j] = key0 + j < n;
      s[j] = valid[j] ? s[j] : kNegInf;
      bm = fmaxf(bm, s[j]);
    }
    bm = fmaxf(bm, swap_rows16(bm));
    bm = fmaxf(bm, swap_halves32(bm));
    const float bms = bm * qk_scale;
    if (bms > m + kRescale) {
      const float al = exp2_fast(m - bms);
      l *= al;
#pragma unroll
      for (int t = 0; t < NH; ++t) o[t] *= al;
      m = bms;
    }
    s16x4_t p_hi, p_lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p = exp2_fast(fmaf(s[j], qk_scale, -m));
      p = valid[j] ? p : 0.f;
      l += p;
      const unsigned short h = bf16_bits(p);
      p_hi[j] = (short)h;
      p_lo[j] = (short)bf16_bits(p - bf16_value(h));
    }
    // V^T fragments: dim 16t + col, keys 4 grp .. +3 (masked keys read as zero)
    const unsigned short* vsh = sm.v[wave];
#pragma unroll
    for (int t = 0; t < NH; ++t) {
      s16x4_t vt;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned short x = vsh[(4 * grp + j) * D + 16 * t + col];
        vt[j] = valid[j] ? (short)x : (short)0;
      }
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, p_hi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, p_lo, o[t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // blocks wave, wave + 4, ...: the next one is always in flight
  const int my = wave < nblk ? (nblk - wave + kWaves - 1) / kWaves : 0;
  Frag f0, f1;
  if (my > 0) load(f0, wave);
  for (int i = 0; i < my; ++i) {
    if (i + 1 < my) load(f1, wave + (i + 1) * kWaves);
    compute(f0, wave + i * kWaves);
    f0 = f1;
  }

  // merge the key groups' partial sums, then the waves through LDS
  l += swap_rows16(l);
  l += swap_halves32(l);
#pragma unroll
  for (int t = 0; t < NH; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.o[wave][16 * t + 4 * grp + j][col] = o[t][j];
  if (grp == 0) {
    sm.m[wave][col] = m;
    sm.l[wave][col] = l;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kTileRows * D; idx += 64 * kWaves) {
    const int rr = idx / D;
    const int d = idx % D;
    const int rg = tile * kTileRows + rr;
    if (rg >= R) continue;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][rr]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.m[w][rr];
      const float f = (mw == kNegInf) ? 0.f : exp2_fast(mw - mx);
      A = fmaf(f, sm.o[w][d][rr], A);
      L = fmaf(f, sm.l[w][rr], L);
    }
    const int i = rg / G;
    const int h = g * G + rg % G;
    const size_t oi = ((size_t)row * a.n_q + i) * a.H_q + h;
    a.out[oi * D + d] = L > 0.f ? A / L : 0.f;
    if (a.lse != nullptr && d == 0) a.lse[oi] = L > 0.f ? (mx + __log2f(L)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_mq(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype != PA_BF16) return hipErrorNotSupported;
  const int rows = a.n_q * (a.H_q / a.H_kv);
  dim3 grid((rows + kTileRows - 1) / kTileRows, a.H_kv, a.batch);
  switch (a.D) {
    case 32:
      hipLaunchKernelGGL(mq_paged_mfma_kernel<32>, grid, dim3(64 * kWaves), 0, stream, a);
      break;
    case 64:
      hipLaunchKernelGGL(mq_paged_mfma_kernel<64>, grid, dim3(64 * kWaves), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(mq_paged_mfma_kernel<128>, grid, dim3(64 * kWaves), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
