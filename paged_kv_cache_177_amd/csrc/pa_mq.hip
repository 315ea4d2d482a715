// Multi-query paged attention on the gfx950 matrix cores: many queries per row attend to the row's
// ragged keys, read through its block table from the same 16-token block pool (cortex-engine
// write-up, kernels section: latent queries cross-attend to a variable number of spike tokens, with
// a FlashAttention-2 style online softmax; a fully masked row gives zeros).
//
// Query "rows" of KV head g are the (query i, head h) pairs with h in g's group: r = i * G + (h - gG).
// One workgroup (4 waves) takes 16 query rows of one (row b, KV head g); its waves split the row's
// 16-token key blocks round-robin (two blocks in flight per wave while one is computed) and merge
// through LDS at the end. Per block, per wave:
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
#include <type_traits>

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
constexpr int kXcds = 8;  // accelerator dies of the chip, each with its own L2

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
  int kept[kWaves][64];                  // block-sparse: each wave's kept blocks of its window
  float o[kWaves][D][kTileRows];
  float m[kWaves][kTileRows];
  float l[kWaves][kTileRows];
};

template <int D, bool SPARSE>
// D = 32 (the latent cross-attention shape) is held to 7 waves per SIMD (72 registers, no spills):
// nearly a whole launch of that workload is resident at once. (8 waves spill; measured slower.)
__attribute__((amdgpu_waves_per_eu(D == 32 ? 7 : 1)))
__global__ __launch_bounds__(64 * kWaves) void mq_paged_mfma_kernel(const DecodeArgs a) {
  constexpr int KC = D / 32;  // k-steps of the score product
  constexpr int NH = D / 16;  // dim tiles of the output product
  __shared__ MqSmem<D> sm;
  int tile, g, row;
  {
    // Workgroups are dealt to the 8 XCDs round-robin by index. All query tiles of one (row, KV
    // head) read the same keys and values, so they are numbered to land on one XCD, where the
    // first tile's reads leave the blocks in that XCD's L2 for the others.
    const int T = (int)a.mq_tiles;
    const int P = a.batch * a.H_kv;
    const int L = (int)blockIdx.x;
    int pair;
    if (P % kXcds == 0) {
      const int q = L / kXcds;
      tile = q % T;
      pair = (q / T) * kXcds + L % kXcds;
    } else {
      tile = L % T;
      pair = L / T;
    }
    row = pair / a.H_kv;
    g = pair % a.H_kv;
  }
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
  // issue the loads of one block (physical id pb, already clamped into the pool)
  auto load = [&](Frag& f, int pb) {
    const size_t base = ((size_t)pb * a.H_kv + g) * (size_t)(kBlock * D);
    const __bf16* kb = kbase + base + (size_t)col * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c) f.k[c] = *reinterpret_cast<const u32x4_t*>(kb + 32 * c);
    const __bf16* vb = vbase + base + (size_t)lane * 8;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) f.v[c] = *reinterpret_cast<const u32x4_t*>(vb + 512 * c);
  };
  // One block: scores, online-softmax update, output product. MASK (the row's partial last block
  // only) drops the keys at or past n: their slots may hold anything, NaN included.
  auto compute = [&](auto mask_tag, const Frag& f, int blk, int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      valid[j] = !MASK || key0 + j < n;
      if (MASK) s[j] = valid[j] ? s[j] : kNegInf;
    }
    // The running max of a query is shared by its four key groups (lanes col + 16 grp). It is
    // raised, to the block maximum over all 16 keys, only when some lane's own keys beat it by
    // more than kRescale; otherwise the block needs no cross-lane step at all.
    const float lm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__builtin_amdgcn_ballot_w64(lm * qk_scale > m + kRescale) != 0) {
      float bm = fmaxf(lm, swap_rows16(lm));
      bm = fmaxf(bm, swap_halves32(bm));
      const float bms = bm * qk_scale;
      if (bms > m + kRescale) {
        const float al = exp2_fast(m - bms);
        l *= al;
#pragma unroll
        for (int t = 0; t < NH; ++t) o[t] *= al;
        m = bms;
      }
    }
    s16x4_t p_hi, p_lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p = exp2_fast(fmaf(s[j], qk_scale, -m));
      if (MASK) p = valid[j] ? p : 0.f;  // a zero scale would make -inf * 0 a NaN
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
        vt[j] = (!MASK || valid[j]) ? (short)x : (short)0;
      }
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, p_hi, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, p_lo, o[t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };
  // full blocks take the unmasked form; the row's partial last block the masked one
  auto step = [&](const Frag& f, int blk, int n) {
    if ((blk + 1) * kBlock <= n)
      compute(std::false_type{}, f, blk, n);
    else
      compute(std::true_type{}, f, blk, n);
  };

  // This wave's blocks are wave, wave + 4, ...; they are taken in windows of up to 64, whose block
  // ids one load brings in (one per lane; the first window's is issued before the row length is
  // known: the table row always has bt_stride entries). A ring of three fragments keeps two blocks
  // in flight while one is computed; the ring is unrolled so no fragment is copied, and every load
  // is issued unconditionally (past the window's end it re-reads the window's last block, which is
  // already cached, and the compute is skipped), so each wait covers exactly the fragment it needs.
  auto window_ids = [&](int w0, int cnt) {
    const int e = w0 + (lane < cnt ? lane : cnt - 1);
    const int idx = wave + e * kWaves;
    const int pb = bt[idx < a.bt_stride ? idx : a.bt_stride - 1];
    return (unsigned)pb < (unsigned)a.num_blocks ? pb : 0;
  };
  // block-sparse: this tile's keep flags (one per 16-token key block); all rows of a 16-row tile
  // belong to one block of 16 queries, tile / G
  const uint8_t* keep_row = nullptr;
  if constexpr (SPARSE) {
    const int n_qb = (a.n_q + kTileRows - 1) / kTileRows;
    keep_row = a.block_mask + ((size_t)row * n_qb + tile / G) * a.mask_kv_blocks;
  }
  auto window_keep = [&](int w0, int cnt) {
    const int idx = wave + (w0 + lane) * kWaves;
    return lane < cnt && idx < a.mask_kv_blocks && keep_row[idx] != 0;
  };
  int ids = window_ids(0, 64);
  bool keep0 = false;
  if constexpr (SPARSE) keep0 = window_keep(0, 64);
  const int n = clampi(a.kv_lens[row], 0, a.max_kv_len);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int my = wave < nblk ? (nblk - wave + kWaves - 1) / kWaves : 0;
  for (int w0 = 0; w0 < my; w0 += 64) {
    const int cnt = my - w0 < 64 ? my - w0 : 64;
    if (w0 > 0) ids = window_ids(w0, cnt);
    // the window's blocks to visit, in order: all of them, or (block-sparse) the kept ones,
    // compacted so that lane j holds the window position of the j-th kept block
    int nv = cnt;
    int pos = lane;
    if constexpr (SPARSE) {
      const bool k = (w0 > 0 ? window_keep(w0, cnt) : keep0) && lane < cnt;
      const unsigned long long kept = __builtin_amdgcn_ballot_w64(k);
      nv = __builtin_popcountll(kept);
      const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(kept >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((unsigned)kept, 0));
      if (k) sm.kept[wave][rank] = lane;
      __builtin_amdgcn_wave_barrier();
      pos = lane < nv ? sm.kept[wave][lane] : 0;
      __builtin_amdgcn_wave_barrier();
      if (nv == 0) continue;
    }
    auto pos_at = [&](int j) {
      const int jj = j < nv ? j : nv - 1;
      return SPARSE ? __builtin_amdgcn_readlane(pos, jj) : jj;
    };
    auto id_at = [&](int j) { return __builtin_amdgcn_readlane(ids, pos_at(j)); };
    auto blk_at = [&](int j) { return wave + (w0 + pos_at(j)) * kWaves; };
    Frag f0, f1, f2;
    load(f0, id_at(0));
    load(f1, id_at(1));
    for (int j = 0; j < nv; j += 3) {
      load(f2, id_at(j + 2));
      step(f0, blk_at(j), n);
      load(f0, id_at(j + 3));
      if (j + 1 < nv) step(f1, blk_at(j + 1), n);
      load(f1, id_at(j + 4));
      if (j + 2 < nv) step(f2, blk_at(j + 2), n);
    }
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

template <bool SPARSE>
hipError_t launch_mq(const DecodeArgs& b, dim3 grid, hipStream_t stream) {
  switch (b.D) {
    case 32:
      hipLaunchKernelGGL((mq_paged_mfma_kernel<32, SPARSE>), grid, dim3(64 * kWaves), 0, stream, b);
      break;
    case 64:
      hipLaunchKernelGGL((mq_paged_mfma_kernel<64, SPARSE>), grid, dim3(64 * kWaves), 0, stream, b);
      break;
    case 128:
      hipLaunchKernelGGL((mq_paged_mfma_kernel<128, SPARSE>), grid, dim3(64 * kWaves), 0, stream,
                         b);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mq(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype != PA_BF16) return hipErrorNotSupported;
  const int rows = a.n_q * (a.H_q / a.H_kv);
  DecodeArgs b = a;
  b.mq_tiles = (rows + kTileRows - 1) / kTileRows;
  const long long wgs = (long long)b.mq_tiles * a.H_kv * a.batch;
  if (wgs * 64 * kWaves > 0xffffffffLL) return hipErrorInvalidValue;  // grid x holds < 2^32 threads
  const dim3 grid((unsigned)wgs);
  return b.block_mask != nullptr ? launch_mq<true>(b, grid, stream)
                                 : launch_mq<false>(b, grid, stream);
}

}  // namespace pa
