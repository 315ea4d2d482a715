// Multi-query paged attention on the gfx950 matrix cores: many queries per row attend to the row's
// ragged keys, read through its block table from the same 16-token block pool (cortex-engine
// write-up, kernels section: latent queries cross-attend to a variable number of spike tokens, with
// a FlashAttention-2 style online softmax; a fully masked row gives zeros).
//
// Query "rows" of KV head g are the (query i, head h) pairs with h in g's group: r = i * G + (h - gG).
// One workgroup (4 waves) takes 16 QT query rows of one (row b, KV head g); its waves split the
// row's 16-token key blocks round-robin (two blocks in flight per wave while one is computed) and
// merge through LDS at the end. Each wave carries the QT sub-tiles of 16 query rows through every
// block it reads, so a block's loads, its V staging and its V^T fragments serve 16 QT queries.
// Per block, per wave and sub-tile:
//   S^T[16 keys][16 q] = K[16 keys][D] . Q^T[D][16 q]   v_mfma_f32_16x16x32_bf16, D/32 steps
//       K is the A operand straight from the block (lane: key l%16, 8 dims), Q^T the B operand
//       (lane: query l%16, 8 dims); the result puts query l%16 in lane l, keys 4(l/16)..+3.
//   online softmax per query: lane-local, plus two cross-lane steps for the block maximum;
//   O^T[D][16 q] += V^T[D][16 keys] . P^T[16 keys][16 q]   v_mfma_f32_16x16x32_bf16, D/16 steps
//       P is split into bf16 hi + lo parts, so the weights keep ~16 bits, and both parts go
//       through one K = 32 product: each lane's B operand is its 4 hi weights then its 4 lo
//       weights, in the lanes where the first product left them (query l%16, keys 4(l/16)..);
//       the A operand holds V^T (lane: dim l%16, keys 4(l/16)..) twice over, read from the block
//       staged in LDS by two ds_read_b64_tr_b16 per 16 dims (the gfx950 transposing LDS read).
// Query rows therefore sit in the same lanes in S^T and O^T: rescales and the final division are
// lane-local.
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
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

// Two fp32 weights -> their bf16 hi parts (RNE, one packed conversion) and the bf16 of what the
// hi parts leave over: p ~ hi + lo to ~16 bits. The remainders p - hi come exactly (both terms are
// within one bf16 step of each other, so the difference is an fp32 number) from the bf16 dot
// product of the hi pair with (-1, 0), resp. (0, -1), accumulated onto p: one instruction each.
// neg0 and neg1 are those two pairs, passed in scalar registers: written as a constant, the first
// pair is encoded as the inline constant -1.0, which this instruction reads as the fp32 -1.0, i.e.
// the pair (0, -1).
__device__ __forceinline__ void split_bf16x2(float p0, float p1, unsigned neg0, unsigned neg1,
                                             unsigned& hi, unsigned& lo) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t));
  const bf16x2_t h = __builtin_bit_cast(bf16x2_t, hi);
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, neg0), p0, false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, neg1), p1, false);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2_t));
}

// A raw-buffer resource for one K or V block: the block's base address in scalar registers, so a
// load adds only the lane's 32-bit offset (the loop-invariant vector offsets need no copies or
// 64-bit address arithmetic per block). Word 3 is the gfx9-family raw-buffer format word; the
// range is wider than any offset used (offsets stay inside the block).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}

// ds_read_b64_tr_b16: within each 16-lane quarter-wave, lanes 4j .. 4j + 3 name (with 8-byte
// addresses, 4 elements each) row j of a 4 x 16 block of 16-bit elements, and lane l receives
// element l of rows 0 .. 3.
__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(
          (__attribute__((address_space(3))) const unsigned short*)p));
}

// a query row's D outputs are contiguous in the merge area, padded so that rows start 16 bytes apart
// on different banks
template <int D>
constexpr int kORow = D + 4;

template <int D, int QT>
struct MqSmem {
  unsigned short v[kWaves][kBlock * D];  // each wave's staged V block
  int kept[kWaves][64];                  // block-sparse: each wave's kept blocks of its window
  float o[kWaves][QT][kTileRows][kORow<D>];
  float m[kWaves][QT][kTileRows];
  float l[kWaves][QT][kTileRows];
};

// query sub-tiles per wave: two for the dense D = 32 kernel (the latent cross-attention shape);
// one elsewhere (the block-sparse skip decision is per block of 16 queries, and wider heads would
// need too many registers)
template <int D, bool SPARSE>
constexpr int mq_qt() { return (D == 32 && !SPARSE) ? 2 : 1; }

// K/V block fragments per wave (RING - 1 blocks in flight while one is computed): three for the
// dense kernels (the D = 32 one, the latent cross-attention shape, may take PA_MQ_RING_D32; its 4
// waves per SIMD allow up to 128 registers). The block-sparse D = 32 kernel keeps two: it computes
// only the kept blocks (about a tenth on the latent workload), and two fragments hold it to 64
// registers, so its launch of 8 waves per SIMD is resident at once (three need 71: 7 waves).
#ifndef PA_MQ_RING_D32
#define PA_MQ_RING_D32 3
#endif
template <int D, bool SPARSE>
constexpr int mq_ring() { return D != 32 ? 3 : (SPARSE ? 2 : PA_MQ_RING_D32); }

template <int D, bool SPARSE>
// D = 32 (the latent cross-attention shape) keeps several waves per SIMD: 8 with one sub-tile (64
// registers), 4 with two (128); a whole launch of that workload is then resident at once.
__attribute__((amdgpu_waves_per_eu(D == 32 ? (mq_qt<D, SPARSE>() == 2 ? 4 : 8) : 1)))
__global__ __launch_bounds__(64 * kWaves) void mq_paged_mfma_kernel(const DecodeArgs a) {
  constexpr int KC = D / 32;  // k-steps of the score product
  constexpr int NH = D / 16;  // dim tiles of the output product
  constexpr int QT = mq_qt<D, SPARSE>();
  constexpr int RING = mq_ring<D, SPARSE>();
  constexpr int TR = kTileRows * QT;  // query rows of a workgroup
  __shared__ MqSmem<D, QT> sm;
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
  const int col = lane & 15;  // query row inside a sub-tile (S^T / O^T column)
  const int grp = lane >> 4;  // key group: keys 4*grp .. 4*grp+3 of a block
  const int G = a.H_q / a.H_kv;
  // query row r -> (query r / G, head r % G of the group): shifts when G is a power of two (a
  // uniform branch), else the divisions
  const bool g_pow2 = (G & (G - 1)) == 0;
  const int g_shift = __builtin_ctz((unsigned)G);
  auto split_row = [&](int r, int& qi, int& hg) {
    if (g_pow2) {
      qi = r >> g_shift;
      hg = r & (G - 1);
    } else {
      qi = r / G;
      hg = r - qi * G;
    }
  };
  const int R = a.n_q * G;  // query rows of this KV head

  // Q^T fragments (B operand) of sub-tile u: query row tile * TR + 16 u + col, dims 32c + 8 grp
  // .. +7; zero for rows past R
  bf16x8_t qf[QT][KC];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int r = tile * TR + kTileRows * u + col;
    const bool row_ok = r < R;
    int qi = 0, hg = 0;
    if (row_ok) split_row(r, qi, hg);
    const int qh = g * G + hg;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (size_t)row * a.q_row_stride +
                       ((size_t)qi * a.H_q + qh) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (row_ok) x = *reinterpret_cast<const u32x4_t*>(qp + 32 * c);
      qf[u][c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  const int* bt = a.block_tables + (size_t)row * a.bt_stride;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v);
  const float qk_scale = a.scale * kLog2e;
  const float inv_qk = 1.0f / qk_scale;  // the raise threshold needs no exact division

  // Per sub-tile: running max m (log2 units), its raise threshold in raw score units thr = (m +
  // kRescale) / qk_scale (recomputed only when m moves), the output accumulators, and the row sums
  // of P, which the matrix cores accumulate with the output: a constant A operand whose first row
  // is all ones turns P^T into sum_k P[q][k] in element 0 of lanes 0 .. 15 (query = lane).
  float m[QT], thr[QT];
  f32x4_t o[QT][NH], ls[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    m[u] = kNegInf;
    thr[u] = kNegInf;
    ls[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NH; ++t) o[u][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const short one = col == 0 ? (short)0x3F80 : (short)0;  // bf16 1.0 in row 0 of the A operand
  const s16x4_t ones = {one, one, one, one};
  const bf16x8_t ones8 =
      __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ones, ones, 0, 1, 2, 3, 0, 1, 2, 3));
  // (-1, 0) and (0, -1) as bf16 pairs in scalar registers (see split_bf16x2)
  unsigned neg0 = 0x0000BF80u, neg1 = 0xBF800000u;
  asm("" : "+s"(neg0), "+s"(neg1));
  // this lane's address for the transposed V^T reads: key 4 grp + col / 4, dims 4 (col % 4) ..
  const unsigned short* vtr = sm.v[wave] + (4 * grp + col / 4) * D + 4 * (col % 4);
  // the same address again, which the compiler cannot prove equal: the second transposed read fills
  // the other half of the A operand (a register copy of the first read would cost 2 VALU per tile)
  int vtr_zero = 0;
  asm("" : "+v"(vtr_zero));
  const unsigned short* vtr2 = vtr + vtr_zero;

  // K fragment (A operand): key col of the block, dims 32c + 8 grp; V: 16 contiguous bytes per lane
  // at lane * 8 elements (its transpose is read back from LDS)
  struct Frag {
    u32x4_t k[KC];
    u32x4_t v[D / 32];
  };
  // issue the loads of one block (physical id pb, already clamped into the pool): buffer loads off a
  // per-block scalar resource with the lanes' fixed 32-bit byte offsets
  const int k_off0 = (col * D + 8 * grp) * 2;
  const int v_off0 = lane * 16;
  auto load = [&](Frag& f, int pb) {
    const size_t base = ((size_t)pb * a.H_kv + g) * (size_t)(kBlock * D);
    const __amdgpu_buffer_rsrc_t kr = block_rsrc(kbase + base);
    const __amdgpu_buffer_rsrc_t vr = block_rsrc(vbase + base);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      f.k[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off0, 64 * c, 0));
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      f.v[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off0, 1024 * c, 0));
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

    const int key0 = blk * kBlock + 4 * grp;
    bool valid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) valid[j] = !MASK || key0 + j < n;
    // V^T fragments (dim 16t + col, keys 4 grp .. +3; masked keys read as zero), shared by the
    // sub-tiles; read now so that the LDS latency hides behind the score products
    s16x4_t vt[NH], vt2[NH];
#pragma unroll
    for (int t = 0; t < NH; ++t) {
      vt[t] = lds_read_tr16(vtr + 16 * t);
      vt2[t] = lds_read_tr16(vtr2 + 16 * t);
    }
    // The sub-tiles' chains run side by side (their products, maxima, exponentials and
    // conversions interleave), with one branch for the rare raise of a running max.
    f32x4_t s[QT];
    float lm[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      s[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c)
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.k[c]),
                                                       qf[u][c], s[u], 0, 0, 0);
    }
    // lanes (of any sub-tile) whose own keys call for a raise; the masks are combined in scalar
    // registers, so the branch takes no vector instruction
    unsigned long long raise = 0;
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      if (MASK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s[u][j] = valid[j] ? s[u][j] : kNegInf;
      }
      // The running max of a query is shared by its four key groups (lanes col + 16 grp). It is
      // raised, to the block maximum over all 16 keys, only when some lane's own keys beat it by
      // more than kRescale; otherwise the block needs no cross-lane step at all.
      lm[u] = fmaxf(fmaxf(s[u][0], s[u][1]), fmaxf(s[u][2], s[u][3]));
      raise |= __builtin_amdgcn_ballot_w64(lm[u] > thr[u]);
    }
    if (raise != 0) {
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        float bm = fmaxf(lm[u], swap_rows16(lm[u]));
        bm = fmaxf(bm, swap_halves32(bm));
        const float bms = bm * qk_scale;
        if (bms > m[u] + kRescale) {
          const float al = exp2_fast(m[u] - bms);
          ls[u][0] *= al;  // the row sums live in element 0 (the other elements are zero)
#pragma unroll
          for (int t = 0; t < NH; ++t) o[u][t] *= al;
          m[u] = bms;
          thr[u] = (bms + kRescale) * inv_qk;
        }
      }
    }
    s16x4_t p_hi[QT], p_lo[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = exp2_fast(fmaf(s[u][j], qk_scale, -m[u]));
        if (MASK) p[j] = valid[j] ? p[j] : 0.f;  // a zero scale would make -inf * 0 a NaN
      }
      unsigned h01, h23, l01, l23;
      split_bf16x2(p[0], p[1], neg0, neg1, h01, l01);
      split_bf16x2(p[2], p[3], neg0, neg1, h23, l23);
      p_hi[u] = __builtin_bit_cast(s16x4_t, u32x2_t{h01, h23});
      p_lo[u] = __builtin_bit_cast(s16x4_t, u32x2_t{l01, l23});
    }
    // k 0..3 of a lane's group carry the hi weights, k 4..7 the lo weights of the same keys
    bf16x8_t pb[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      pb[u] = __builtin_bit_cast(bf16x8_t,
                                 __builtin_shufflevector(p_hi[u], p_lo[u], 0, 1, 2, 3, 4, 5, 6, 7));
      ls[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb[u], ls[u], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NH; ++t) {
      if (MASK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vt[t][j] = valid[j] ? vt[t][j] : (short)0;
          vt2[t][j] = valid[j] ? vt2[t][j] : (short)0;
        }
      }
      const bf16x8_t va =
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vt[t], vt2[t], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int u = 0; u < QT; ++u)
        o[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[u], o[u][t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // This wave's blocks are wave, wave + 4, ...; they are taken in windows of up to 64, whose block
  // ids one load brings in (one per lane; the first window's is issued before the row length is
  // known: the table row always has bt_stride entries). A ring of RING fragments keeps RING - 1
  // blocks in flight while one is computed; the ring is unrolled so no fragment is copied, and
  // every load is issued unconditionally (past the window's end it re-reads the window's last
  // block, which is already cached, and the compute is skipped), so each wait covers exactly the
  // fragment it needs.
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
  // The loop below takes only full blocks, so it runs the unmasked compute alone; the row's
  // partial last block (if any) is done after it by the wave that owns it.
  const int nfull = n / kBlock;
  const int my = wave < nfull ? (nfull - wave + kWaves - 1) / kWaves : 0;
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
    Frag f[RING];
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r) load(f[r], id_at(r));
    for (int j = 0; j < nv; j += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        // the slot computed one step ago takes the block RING - 1 ahead
        load(f[(r + RING - 1) % RING], id_at(j + r + RING - 1));
        if (r == 0 || j + r < nv) compute(std::false_type{}, f[r], blk_at(j + r), n);
      }
    }
  }
  if (n % kBlock != 0 && nfull % kWaves == wave) {
    // the partial last block, block nfull of the row (block-sparse: only if its tile keeps it)
    bool take = true;
    if constexpr (SPARSE) take = nfull < a.mask_kv_blocks && keep_row[nfull] != 0;
    if (take) {
      const int pb = bt[nfull < a.bt_stride ? nfull : a.bt_stride - 1];
      Frag f;
      load(f, (unsigned)pb < (unsigned)a.num_blocks ? pb : 0);
      compute(std::true_type{}, f, nfull, n);
    }
  }

  // merge the waves through LDS: each wave parks its rows' outputs (a query row's D values
  // contiguous), maxima and sums
#pragma unroll
  for (int u = 0; u < QT; ++u) {
#pragma unroll
    for (int t = 0; t < NH; ++t)
      *reinterpret_cast<f32x4_t*>(&sm.o[wave][u][col][16 * t + 4 * grp]) = o[u][t];
    if (grp == 0) {
      sm.m[wave][u][col] = m[u];
      sm.l[wave][u][col] = ls[u][0];
    }
  }
  __syncthreads();
  // TPR threads per query row, DPT consecutive dims each: a row's weights and normaliser are
  // formed once per thread, not once per output element
  constexpr int TPR = 64 * kWaves / TR;
  constexpr int DPT = D / TPR;
  static_assert(TPR * TR == 64 * kWaves && DPT * TPR == D && DPT % 2 == 0, "merge layout");
  const int rr = threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * DPT;
  const int u = rr / kTileRows;
  const int c = rr % kTileRows;
  const int rg = tile * TR + rr;
  if (rg < R) {
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][u][c]);
    float fw[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.m[w][u][c];
      fw[w] = (mw == kNegInf) ? 0.f : exp2_fast(mw - mx);
      L = fmaf(fw[w], sm.l[w][u][c], L);
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    float A[DPT];
#pragma unroll
    for (int k = 0; k < DPT; ++k) A[k] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
#pragma unroll
      for (int k = 0; k < DPT; k += 2) {
        const f32x2_t x = *reinterpret_cast<const f32x2_t*>(&sm.o[w][u][c][d0 + k]);
        A[k] = fmaf(fw[w], x[0], A[k]);
        A[k + 1] = fmaf(fw[w], x[1], A[k + 1]);
      }
    }
    int i, hg;
    split_row(rg, i, hg);
    const int h = g * G + hg;
    const size_t oi = ((size_t)row * a.n_q + i) * a.H_q + h;
    float* op = a.out + oi * D + d0;
#pragma unroll
    for (int k = 0; k < DPT; k += 2) *reinterpret_cast<f32x2_t*>(op + k) = {A[k] * inv, A[k + 1] * inv};
    if (a.lse != nullptr && d0 == 0) a.lse[oi] = L > 0.f ? (mx + __log2f(L)) * kLn2 : kNegInf;
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

// query rows per workgroup of the kernel instantiation a launch will use
int mq_tile_rows(int D, bool sparse) {
  if (sparse) return kTileRows * (D == 32 ? mq_qt<32, true>() : D == 64 ? mq_qt<64, true>()
                                                                        : mq_qt<128, true>());
  return kTileRows * (D == 32 ? mq_qt<32, false>() : D == 64 ? mq_qt<64, false>()
                                                             : mq_qt<128, false>());
}

}  // namespace

hipError_t launch_decode_mq(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype != PA_BF16) return hipErrorNotSupported;
  const int rows = a.n_q * (a.H_q / a.H_kv);
  DecodeArgs b = a;
  const int tr = mq_tile_rows(a.D, a.block_mask != nullptr);
  b.mq_tiles = (rows + tr - 1) / tr;
  const long long wgs = (long long)b.mq_tiles * a.H_kv * a.batch;
  if (wgs * 64 * kWaves > 0xffffffffLL) return hipErrorInvalidValue;  // grid x holds < 2^32 threads
  const dim3 grid((unsigned)wgs);
  return b.block_mask != nullptr ? launch_mq<true>(b, grid, stream)
                                 : launch_mq<false>(b, grid, stream);
}

}  // namespace pa
