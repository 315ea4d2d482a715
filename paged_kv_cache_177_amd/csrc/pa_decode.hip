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
// Mapping (one workgroup of kWaves waves per chunk (KV head g, row b, split s)):
//   * A row is cut into chunks of chunk_tokens(D) tokens; split s owns chunk s. The workgroup
//     covers the G = H_q / H_kv query heads of KV head g, so each K/V byte is loaded once and
//     feeds all G heads from registers.
//   * A wave works one 16-token block per step. Every lane owns 8 dims (16 bytes of bf16) of
//     TPL = D/32 of the block's tokens, so each 16-byte-per-lane load instruction reads one
//     contiguous 1 KB run of the block: fully coalesced, non-temporal (K/V are read once), with a
//     wave-uniform block base and a lane offset. Blocks of the chunk are dealt round-robin to the
//     waves; each wave keeps its next block in flight while it computes the current one.
//   * q.k: packed bf16 dot products (v_dot2_f32_bf16) accumulate in fp32, then a DPP butterfly
//     over the LPT = D/8 lanes of a token. Scores are kept in log2 units (scale * log2(e) folded
//     in) so the softmax uses the hardware exp2.
//   * Online softmax per lane: each lane keeps a running max m, sum l and an 8-dim accumulator
//     per head for the tokens it sees. m is raised only when a score exceeds it by more than 8
//     (log2 units), so rescales are rare; weights stay <= 2^8 and the result is exact up to
//     rounding. Only a chunk's partial last block runs the masked update.
//   * At the end the lanes' streams are merged to a common max (DPP inside 16-lane rows, a
//     swizzle across rows, a swap across half-waves), then the waves through LDS. One split
//     writes out/lse; several write normalised partials plus their log-sum-exp. When no row of
//     the launch has more than 16 splits, the split grid merges them itself: the workgroup that
//     finishes a (row, KV head)'s last split merges its heads (see merge_if_last); otherwise
//     lse_reduce_kernel runs after the launch. Both merges give the same bits.
//   * Three launch shapes run the same chunks: a grid of one workgroup per (g, b, s) whose
//     workgroups past a row's last split exit at once; for rows long enough for many splits, a
//     compact grid whose workgroups map to the chunks through the rows' lengths (batches of at
//     most 64 rows), or a persistent grid that pulls chunks from a counter (see
//     decode_persistent_kernel).
//   * Either can also do the append (the fused call): the wave whose blocks include a row's new
//     token stores its key (rotated) and value before it loads that block, and every workgroup
//     rotates its queries in registers, with the append kernel's arithmetic, so the results are
//     those of the separate append and decode bit for bit.
#include "pa_internal.h"

#include <map>
#include <type_traits>
#include <mutex>
#include <tuple>

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_PERSISTENT
#define PA_DECODE_PERSISTENT 1
#endif
// Rows long enough for the persistent kernel, in a batch of at most 64 rows: 1 = a compact grid
// instead (see decode_vector_kernel), 0 = the persistent kernel.
#ifndef PA_DECODE_COMPACT
#define PA_DECODE_COMPACT 1
#endif
// 1 = the split grid merges the splits of rows with at most 16 splits itself (no second launch);
// 0 = lse_reduce_kernel always does.
#ifndef PA_DECODE_GRID_MERGE
#define PA_DECODE_GRID_MERGE 1
#endif
// 1 = a bf16 split grid larger than the device holds hands out its last chunks by tickets (see
// take_ticket); 0 = every chunk has a fixed workgroup.
#ifndef PA_DECODE_TICKETS
#define PA_DECODE_TICKETS 1
#endif

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 units
constexpr int kWaves = PA_DECODE_WAVES;
constexpr float kNegInf = -__builtin_inff();
constexpr int kTicketExtraRows = 32;  // ticketed grid rows beyond the chunks they share

// ---- cross-lane helpers -----------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i inside each 8-lane half row
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i inside each 16-lane row
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return dpp<0x120 + N>(x);
}

// Sum over the LPT consecutive lanes that share one token (result in all of them).
template <int LPT>
__device__ __forceinline__ float token_lane_sum(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lanes per token");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (LPT >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (LPT >= 16) x += dpp<kRowMirror>(x);
  return x;
}

// Reduce over the token streams inside one 16-lane row (lanes congruent mod LPT).
template <int LPT, bool MAX>
__device__ __forceinline__ float row_stream_reduce(float x) {
  if constexpr (LPT <= 4) x = MAX ? fmaxf(x, row_ror<4>(x)) : x + row_ror<4>(x);
  if constexpr (LPT <= 8) x = MAX ? fmaxf(x, row_ror<8>(x)) : x + row_ror<8>(x);
  return x;
}

// Lane i <-> lane i ^ 16 inside each 32-lane half: ds_swizzle, bit-mask mode
// (and_mask 0x1f, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ float swap_rows16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
// Lane i <-> lane i ^ 32.
__device__ __forceinline__ float swap_halves32(float x) { return __shfl_xor(x, 32); }

template <int LPT, bool MAX>
__device__ __forceinline__ float wave_stream_reduce(float x) {
  x = row_stream_reduce<LPT, MAX>(x);
  x = MAX ? fmaxf(x, swap_rows16(x)) : x + swap_rows16(x);
  x = MAX ? fmaxf(x, swap_halves32(x)) : x + swap_halves32(x);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---- 8 elements of one token (one lane's share) -------------------------------------------------
template <typename T>
struct Vec8;

template <>
struct Vec8<__bf16> {
  uint4 w;
  // K/V are streamed once: non-temporal loads keep them from displacing reused lines in the caches
  __device__ __forceinline__ void load(const __bf16* p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w = make_uint4(x.x, x.y, x.z, x.w);
  }
  __device__ __forceinline__ void load_cached(const __bf16* p) {
    w = *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_f32(float* o) const {
    o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
    o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z); o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
  }
  // round each to bf16 (to nearest even), as the append kernel stores
  __device__ __forceinline__ void from_f32(const float* o) {
    auto pk = [](float lo, float hi) {
      return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo)) |
             ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi)) << 16);
    };
    w = make_uint4(pk(o[0], o[1]), pk(o[2], o[3]), pk(o[4], o[5]), pk(o[6], o[7]));
  }
  __device__ __forceinline__ void store(__bf16* p) const { *reinterpret_cast<uint4*>(p) = w; }
  // <a, b> over the 8 elements: one chain of packed dot products, fp32 accumulation of the
  // exact bf16 products
  __device__ __forceinline__ float dot(const Vec8& b) const {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                              __builtin_bit_cast(bf16x2_t, b.w.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                        __builtin_bit_cast(bf16x2_t, b.w.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                        __builtin_bit_cast(bf16x2_t, b.w.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                        __builtin_bit_cast(bf16x2_t, b.w.w), s, false);
    return s;
  }
};

template <>
struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  // element-wise through native 4-float vectors: whole-struct float4 copies become memory copies
  // that kept the fused append's pieces in scratch memory
  __device__ __forceinline__ void load_cached(const float* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 x = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 y = reinterpret_cast<const f32x4*>(p)[1];
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void to_f32(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  __device__ __forceinline__ void from_f32(const float* o) {
    a = make_float4(o[0], o[1], o[2], o[3]);
    b = make_float4(o[4], o[5], o[6], o[7]);
  }
  __device__ __forceinline__ void store(float* p) const {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    reinterpret_cast<f32x4*>(p)[0] = f32x4{a.x, a.y, a.z, a.w};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{b.x, b.y, b.z, b.w};
  }
  __device__ __forceinline__ float dot(const Vec8& o) const {
    float s0 = a.x * o.a.x;
    float s1 = a.y * o.a.y;
    s0 = fmaf(a.z, o.a.z, s0);
    s1 = fmaf(a.w, o.a.w, s1);
    s0 = fmaf(b.x, o.b.x, s0);
    s1 = fmaf(b.y, o.b.y, s1);
    s0 = fmaf(b.z, o.b.z, s0);
    s1 = fmaf(b.w, o.b.w, s1);
    return s0 + s1;
  }
};

// One block's worth of this lane's K and V (TPL tokens).
template <typename T, int TPL>
struct BlockFrag {
  Vec8<T> k[TPL], v[TPL];
};

// ---- one chunk of one (row, KV head): the unit of work of a workgroup ----------------------------
struct Chunk {
  int row, g, split;
  int tok0, ntok, nblk, tail_blk;  // tail_blk: index of the partial last block, or -1
  int ns;                          // splits of the row (1: write out/lse directly)
  int gap_s, gap_shift;            // padded layout: the row's gap start and width
};

__device__ __forceinline__ Chunk make_chunk(int row, int g, int split, int n, int gap_s,
                                            int gap_shift, int chunk) {
  Chunk ch;
  ch.row = row;
  ch.g = g;
  ch.split = split;
  ch.ns = num_splits(n, chunk);
  ch.tok0 = split * chunk;
  const int rest = n - ch.tok0;
  ch.ntok = rest < chunk ? (rest > 0 ? rest : 0) : chunk;
  ch.nblk = (ch.ntok + kBlock - 1) / kBlock;
  ch.tail_blk = (ch.ntok % kBlock) != 0 ? ch.nblk - 1 : -1;
  ch.gap_s = gap_s;
  ch.gap_shift = gap_shift;
  return ch;
}



// Ordering groups of a row's chunks for the compact and persistent launches: the full chunks
// (splits 0 .. n / chunk - 1) go first, the row's short last chunk (split n / chunk, when there is
// one, or split 0 of an empty row) after every row's full ones.
__device__ __forceinline__ void chunk_groups(int n, int chunk, int* full, int* part) {
  *full = n / chunk;
  *part = (n % chunk != 0 || n == 0) ? 1 : 0;
}

template <int G, int D, int WAVES>
struct EpilogueSmem {
  float acc[WAVES][G][D];
  float m[WAVES][G];
  float l[WAVES][G];
};

// Per-wave machinery shared by the grid and the persistent kernels: loads of queries, block ids
// and K/V blocks, the online-softmax update for one block, and the end-of-chunk merge.
template <typename T, int D, int G, bool PADDED>
struct Worker {
  static constexpr int LPT = D / 8;         // lanes per token
  static constexpr int TPI = 64 / LPT;      // tokens per load instruction
  static constexpr int TPL = kBlock / TPI;  // tokens of a block per lane
  static_assert(TPL >= 1 && TPL * TPI == kBlock, "block/lane geometry");
  using Frag = BlockFrag<T, TPL>;
  using Smem = EpilogueSmem<G, D, kWaves>;

  const DecodeArgs& a;
  const int lane, wave, tr, c;
  const unsigned lane_off;  // this lane's element offset inside a [16][D] block (token tr)
  const float qk_scale;
  const T* __restrict__ kbase;
  const T* __restrict__ vbase;
  Vec8<T> q[G];
  float m[G], l[G], acc[G][8];

  __device__ __forceinline__ explicit Worker(const DecodeArgs& args)
      : a(args),
        lane(threadIdx.x & 63),
        wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        tr((threadIdx.x & 63) / LPT),
        c((threadIdx.x & 63) % LPT),
        lane_off((unsigned)(((threadIdx.x & 63) / LPT) * D + ((threadIdx.x & 63) % LPT) * 8)),
        qk_scale(args.scale * kLog2e),
        kbase(reinterpret_cast<const T*>(args.k)),
        vbase(reinterpret_cast<const T*>(args.v)) {}

  // LDS that a worker needs besides the epilogue's (none for this one)
  template <typename S>
  __device__ __forceinline__ void bind(S&) {}
  // this chunk's queries, from memory or from the chunk's G x D queries staged in LDS
  __device__ __forceinline__ void load_queries(int row, int g) { load_q(q, row, g); }
  __device__ __forceinline__ void load_queries_from(const T* qs) {
#pragma unroll
    for (int h = 0; h < G; ++h) q[h].load_cached(qs + h * D + c * 8);
  }

  // queries of the G heads of KV head g in row `row`: this lane's 8 dims of each
  __device__ __forceinline__ void load_q(Vec8<T>* qq, int row, int g) const {
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)row * a.q_row_stride +
                  (size_t)g * G * D + c * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qq[h].load_cached(qp + (size_t)h * D);
  }

  // block ids of a chunk: lane i holds logical block tok0/16 + i (index clamped into the row's
  // table; entries past the chunk are never used; ids clamped into the pool)
  __device__ __forceinline__ int load_ids(int row, int tok0) const {
    if constexpr (PADDED) {
      return 0;
    } else {
      const int e = (tok0 >> 4) + lane;
      const int v = a.block_tables[(size_t)row * a.bt_stride + (e < a.bt_stride ? e : a.bt_stride - 1)];
      return v;
    }
  }
  __device__ __forceinline__ int clamp_id(int v) const {
    return (unsigned)v < (unsigned)a.num_blocks ? v : 0;
  }

  // ---- append fused into the split kernel ----
  // This lane's 8 cos/sin entries at table row pos: lane c holds dims 8c .. 8c+7, whose
  // rotate-half pair index is (8c + e) mod D/2.
  __device__ __forceinline__ void load_trig(int pos, float* cs, float* sn) const {
    const size_t i0 = (size_t)pos * (D / 2) + (size_t)((c & (LPT / 2 - 1)) * 8);
    const float4* cp = reinterpret_cast<const float4*>(a.cos + i0);
    const float4* sp = reinterpret_cast<const float4*>(a.sin + i0);
    const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w;
    cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
    sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w;
    sn[4] = s1.x; sn[5] = s1.y; sn[6] = s1.z; sn[7] = s1.w;
  }
  // The lane holding dims 8c + D/2 (or 8c - D/2): c ^ (LPT / 2).
  __device__ __forceinline__ int partner() const { return c ^ (LPT / 2); }

  // Rotate-half RoPE of this lane's 8 dims `own`, paired with the partner lane's 8 dims: the low
  // half gives own*cos - partner*sin, the high half own*cos + partner*sin, every product and sum
  // a separate fp32 operation, rounded to T -- the append kernel's arithmetic, bit for bit.
  __device__ __forceinline__ void rope8(const Vec8<T>& own, const Vec8<T>& other, const float* cs,
                                        const float* sn, Vec8<T>& out) const {
#pragma clang fp contract(off)
    float x[8], y[8], r[8];
    own.to_f32(x);
    other.to_f32(y);
    const bool low = c < LPT / 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = x[e] * cs[e];
      const float p1 = y[e] * sn[e];
      r[e] = low ? p0 - p1 : p0 + p1;
    }
    out.from_f32(r);
  }

  // This lane's piece of row `row`'s new key (and its partner half, for the rotation) and
  // value for KV head g: dims 8c .. 8c+7 (read by every wave, since any may store them).
  __device__ __forceinline__ void fused_load(int row, int g, Vec8<T>& kx, Vec8<T>& kp,
                                             Vec8<T>& vx) const {
    const size_t src = ((size_t)row * a.H_kv + g) * D;
    const T* kn = reinterpret_cast<const T*>(a.k_new) + src;
    kx.load_cached(kn + c * 8);
    vx.load_cached(reinterpret_cast<const T*>(a.v_new) + src + c * 8);
    if (a.cos != nullptr) kp.load_cached(kn + partner() * 8);
  }

  // The new token's index t (dest, or positions when dest is NULL) clamped as the append kernel
  // clamps it: into the row's block table (paged) or the row's columns (padded).
  __device__ __forceinline__ int fused_index(int row) const {
    return fused_clamp(a.dest != nullptr ? a.dest[row] : a.positions[row]);
  }
  __device__ __forceinline__ int fused_clamp(int t) const {
    return PADDED ? clampi(t, 0, a.seq_cap - 1) : clampi(t, 0, a.bt_stride * kBlock - 1);
  }

  // Whether this wave stores row ch.row's new token t: only the workgroup whose chunk holds it
  // (the last chunk when it lies outside the row's n valid tokens) and, in it, only the wave
  // whose blocks include it. *first: the token's block is this wave's first block.
  __device__ __forceinline__ bool fused_target(const Chunk& ch, int n, int t, bool* first) const {
    int v = t;  // the token's index among the row's valid tokens, or -1 (a padding column)
    if constexpr (PADDED)
      v = t < ch.gap_s ? t : (t >= ch.gap_s + ch.gap_shift ? t - ch.gap_shift : -1);
    const bool inside = v >= 0 && v < n;
    const int owner = inside ? v / chunk_tokens(D) : ch.ns - 1;
    const int b = inside ? (v - ch.tok0) / kBlock : 0;  // the token's block within the chunk
    *first = inside && b == wave;
    return ch.split == owner && b % kWaves == wave;
  }

  // Store the new key (rotated at pos when the pool has RoPE tables) and value of token t, KV
  // head ch.g, at the slot the append kernel stores it to. Later loads of this wave see the
  // stores (a wave's memory operations stay in order); no other workgroup of the launch reads
  // the slot.
  __device__ __forceinline__ void fused_store(Vec8<T> kx, const Vec8<T>& kp, const Vec8<T>& vx,
                                              const Chunk& ch, int t, int pos) const {
    size_t slot;  // element offset of [.., ch.g, t's slot or column, 0]
    if constexpr (PADDED) {
      slot = (((size_t)ch.row * a.H_kv + ch.g) * a.seq_cap + t) * D;
    } else {
      int blk = a.block_tables[(size_t)ch.row * a.bt_stride + t / kBlock];
      blk = (unsigned)blk < (unsigned)a.num_blocks ? blk : 0;
      slot = (((size_t)blk * a.H_kv + ch.g) * kBlock + (t % kBlock)) * D;
    }
    if (lane >= LPT) return;
    if (a.cos != nullptr) {
      float cs[8], sn[8];
      load_trig(pos, cs, sn);
      rope8(kx, kp, cs, sn, kx);
    }
    kx.store(reinterpret_cast<T*>(const_cast<void*>(a.k)) + slot + c * 8);
    vx.store(reinterpret_cast<T*>(const_cast<void*>(a.v)) + slot + c * 8);
  }

  // Rotate the queries at pos (pools with RoPE tables; each head's partner half is read from
  // qset, the chunk's G x D queries in memory or in LDS) and, in split 0, store them to q_out.
  __device__ __forceinline__ void fused_queries(const Chunk& ch, int pos, const T* qset) {
    if (a.cos != nullptr) {
      float cs[8], sn[8];
      load_trig(pos, cs, sn);
      const T* qp = qset + partner() * 8;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        Vec8<T> other;
        other.load_cached(qp + (size_t)h * D);
        rope8(q[h], other, cs, sn, q[h]);
      }
    }
    if (a.q_out != nullptr && ch.split == 0 && wave == 0 && lane < LPT) {
      T* qo = reinterpret_cast<T*>(a.q_out) + ((size_t)ch.row * a.H_q + (size_t)ch.g * G) * D +
              c * 8;
#pragma unroll
      for (int h = 0; h < G; ++h) q[h].store(qo + (size_t)h * D);
    }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
  }

  __device__ __forceinline__ void load_block(Frag& f, const Chunk& ch, int ids, int blk) const {
    if constexpr (PADDED) {
      const size_t head_base = ((size_t)ch.row * a.H_kv + ch.g) * (size_t)a.seq_cap * D;
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int tv = ch.tok0 + blk * kBlock + tr + j * TPI;
        int col = tv < ch.gap_s ? tv : tv + ch.gap_shift;
        col = col < a.kv_cols ? col : a.kv_cols - 1;
        const size_t off = head_base + (size_t)col * D + c * 8;
        f.k[j].load(kbase + off);
        f.v[j].load(vbase + off);
      }
    } else {
      const int pb = clamp_id(__builtin_amdgcn_readlane(ids, blk));
      const size_t boff = ((size_t)pb * a.H_kv + ch.g) * (size_t)(kBlock * D);
      // uniform block base + a 32-bit lane byte offset: the scalar-base form of the global load
      const char* kb = reinterpret_cast<const char*>(kbase + boff);
      const char* vb = reinterpret_cast<const char*>(vbase + boff);
      unsigned lb = lane_off * (unsigned)sizeof(T);
      // keep the lane offset a 32-bit value at the load, so the compiler cannot hoist a 64-bit
      // widening out of the loop and fall back to vector 64-bit addresses (costing registers)
      asm volatile("" : "+v"(lb));
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const unsigned o = lb + (unsigned)(j * TPI * D * sizeof(T));
        f.k[j].load(reinterpret_cast<const T*>(kb + o));
        f.v[j].load(reinterpret_cast<const T*>(vb + o));
      }
    }
  }

  // Online-softmax update with one block of the chunk. MASK is for the chunk's partial last block:
  // its slots past the chunk end may hold anything (NaN included) and never reach the sums.
  template <bool MASK>
  __device__ __forceinline__ void update(const Frag& f, const Chunk& ch, int blk) {
    bool valid[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) valid[j] = !MASK || blk * kBlock + tr + j * TPI < ch.ntok;
    // raw scores q.k; the scale (times log2 e) is applied to the block maximum and inside the
    // exponent's fused multiply-add
    float s[TPL][G];
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[j][h] = token_lane_sum<LPT>(q[h].dot(f.k[j]));
        if (MASK) s[j][h] = valid[j] ? s[j][h] : kNegInf;
      }
    float smax[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int j = 1; j < TPL; ++j) mx = fmaxf(mx, s[j][h]);
      smax[h] = mx * qk_scale;
      need |= smax[h] > m[h] + kRescale;
    }
    if (need) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = smax[h] > m[h] + kRescale ? smax[h] : m[h];
        const float al = exp2_fast(m[h] - mn);
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      float vf[8];
      f.v[j].to_f32(vf);
      if (MASK) {
        // masked slots may hold anything (NaN included): never let them reach the sums
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = valid[j] ? vf[e] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = exp2_fast(fmaf(s[j][h], qk_scale, -m[h]));
        // a stream that has seen only masked tokens has m = -inf: exp2(-inf - -inf) is NaN
        if (MASK) p = valid[j] ? p : 0.f;
        l[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  __device__ __forceinline__ int blk_of(int i) const { return wave + i * kWaves; }
  __device__ __forceinline__ int my_blocks(const Chunk& ch) const {
    return wave < ch.nblk ? (ch.nblk - wave + kWaves - 1) / kWaves : 0;
  }

  // Stream this wave's `my` blocks (wave, wave + kWaves, ...) of `ch`; the caller has issued the
  // first one into f0. The two fragments swap roles every block (loop unrolled by two), so the next
  // block is always in flight while the current one is computed, with no register copies (copying
  // a fragment would wait for its load). The loads of the steady loop are unconditional, so the
  // wait before each update covers exactly the older fragment. The chunk's partial last block, if
  // this wave owns it (it is then the wave's last block), takes the masked update.
  __device__ __forceinline__ void run_blocks(Frag& f0, Frag& f1, const Chunk& ch, int ids, int my) {
    int i = 0;
    for (; i + 2 < my; i += 2) {
      load_block(f1, ch, ids, blk_of(i + 1));
      update<false>(f0, ch, blk_of(i));
      load_block(f0, ch, ids, blk_of(i + 2));
      update<false>(f1, ch, blk_of(i + 1));
    }
    const bool tail = my > 0 && blk_of(my - 1) == ch.tail_blk;
    if (i + 1 < my) {
      load_block(f1, ch, ids, blk_of(i + 1));
      update<false>(f0, ch, blk_of(i));
      if (tail) update<true>(f1, ch, blk_of(i + 1));
      else update<false>(f1, ch, blk_of(i + 1));
    } else if (i < my) {
      if (tail) update<true>(f0, ch, blk_of(i));
      else update<false>(f0, ch, blk_of(i));
    }
  }

  // Merge the lanes' streams to one (m, l, acc) per wave and park it in LDS (then a barrier).
  __device__ __forceinline__ void merge_to_smem(Smem& sm) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mw = wave_stream_reduce<LPT, true>(m[h]);
      const float f = (m[h] == kNegInf) ? 0.f : exp2_fast(m[h] - mw);
      l[h] = wave_stream_reduce<LPT, false>(l[h] * f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = wave_stream_reduce<LPT, false>(acc[h][e] * f);
      m[h] = mw;
    }
    if (lane < LPT) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.acc[wave][h][c * 8 + e] = acc[h][e];
        if (c == 0) {
          sm.m[wave][h] = m[h];
          sm.l[wave][h] = l[h];
        }
      }
    }
    __syncthreads();
  }

  // Combine the waves' parts and write out/lse (one split) or the split's partial.
  __device__ __forceinline__ void write_result(const Smem& sm, const Chunk& ch) const {
    const int H_q = a.H_kv * G;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kWaves) {
      const int h = idx / D;
      const int d = idx % D;
      float mx = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][h]);
      float A = 0.f, L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.m[w][h];
        const float f = (mw == kNegInf) ? 0.f : exp2_fast(mw - mx);
        A = fmaf(f, sm.acc[w][h][d], A);
        L = fmaf(f, sm.l[w][h], L);
      }
      const float o = L > 0.f ? A / L : 0.f;
      const float lse2 = L > 0.f ? mx + __log2f(L) : kNegInf;
      const int hq = ch.g * G + h;
      if (ch.ns == 1) {
        a.out[((size_t)ch.row * H_q + hq) * D + d] = o;
        if (a.lse != nullptr && d == 0) a.lse[(size_t)ch.row * H_q + hq] = lse2 * kLn2;
      } else {
        const size_t pr = ((size_t)ch.row * H_q + hq) * a.s_max + ch.split;
        if (a.merge_counts != nullptr) {
          // merged in this launch, maybe on another XCD: device-coherent stores (through this
          // XCD's L2), so no cache-wide write-back is needed before the count
          __hip_atomic_store(&a.part_o[pr * D + d], o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (d == 0)
            __hip_atomic_store(&a.part_lse[pr], lse2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          a.part_o[pr * D + d] = o;
          if (d == 0) a.part_lse[pr] = lse2;
        }
      }
    }
  }
};

// ---- the single-query worker on the matrix cores (bf16) -------------------------------------------
// The same chunks, the same dealing of a chunk's blocks to the waves and the same end-of-chunk
// combination as Worker (whose helpers it inherits), with each block's arithmetic on the matrix
// cores. A wave's G query heads are the columns of one 16-column tile (columns G .. 15 are zero), so
// per block and wave:
//   S^T[16 keys][16 q] = K[16 keys][D] . Q^T[D][16 q]      v_mfma_f32_16x16x32_bf16, D/32 steps
//     K is the A operand loaded straight from the block (lane: key l%16, dims 32c + 8(l/16) .. +7),
//     Q^T the B operand (lane: head l%16, the same dims); lane l gets head l%16, keys 4(l/16)..+3.
//   online softmax per head, its running max shared by its four lanes (l%16 + 16k): raised to the
//     block maximum only when some lane's scores beat it by more than kRescale (a wave ballot
//     against a threshold kept in raw score units), so most blocks take no cross-lane step;
//   O^T[D][16 q] += V^T[D][16 keys] . P^T[16 keys][16 q]   D/16 tiles
//     P^T is the first product's result in place; V^T comes from the block staged in the wave's LDS
//     area and read back transposed (ds_read_b64_tr_b16). P enters as two bf16 parts, hi + lo
//     (within 2^-16 of each fp32 weight), and the weight sums come from the same products (a
//     constant A operand whose row 0 is ones): numerator and denominator see the same weights.
//     D <= 64: one v_mfma_f32_16x16x32_bf16 per tile takes both parts (B operand: a lane's 4 hi
//     weights, then its 4 lo weights; A operand: its V^T fragment twice over, from a second
//     transposed read). D = 128: two v_mfma_f32_16x16x16_bf16 per tile (hi, then lo), since the
//     second copy of the 8 tiles' fragments would not fit in 3 waves' registers per SIMD.
// K is loaded as whole 1 KB runs like V (as the products' operand layout it would be half lines of
// 64 bytes, each read by two instructions: 8% slower on the B=128 step) and rearranged through the
// wave's padded K area in LDS.
// A lane keeps its head's outputs for dims 16t + 4(l/16) .. +3, so no lane merge is needed.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Two fp32 weights -> their bf16 parts rounded to nearest (one packed conversion) and the bf16 of
// what those leave over.
__device__ __forceinline__ void split_bf16x2(float p0, float p1, unsigned& hi, unsigned& lo) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t));
  const f32x2_t h = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{p0, p1} - h, bf16x2_t));
}

// ds_read_b64_tr_b16: within each 16-lane quarter-wave, lanes 4j .. 4j + 3 name (8-byte addresses,
// 4 elements each) row j of a 4 x 16 block of 16-bit elements; lane l receives element l of rows
// 0 .. 3.
__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(
          (__attribute__((address_space(3))) const unsigned short*)p));
}

template <int D, int G, bool PADDED>
struct WorkerM : Worker<__bf16, D, G, PADDED> {
  using Base = Worker<__bf16, D, G, PADDED>;
  using Base::a;
  using Base::lane;
  using Base::wave;
  using Base::qk_scale;
  using Base::kbase;
  using Base::vbase;
  static constexpr int KC = D / 32;  // 32-dim steps of the score product
  static constexpr int NH = D / 16;  // 16-dim tiles of the output product
  static constexpr int VC = D / 32;  // 16-byte pieces per lane of a block's V (32 D bytes)
  // the output product as one K = 32 product per tile taking both weight parts (D <= 64), or as
  // two K = 16 products (D = 128, where the doubled V^T operand would not fit the register cap)
  static constexpr bool kK32 = D <= 64;
  static_assert(G <= 16, "a group's heads fill at most one 16-column tile");
  // a block's K and V as loaded: lane l holds elements 8l + 512c .. +7 of each [16][D] array
  // (whole 1 KB runs per load instruction), rearranged through LDS for the products
  struct Frag {
    u32x4_t k[KC];
    u32x4_t v[VC];
  };
  // K rows padded by 8 elements (16 bytes): the 16 lanes of a quarter-wave, reading one 16-byte
  // piece of 16 different rows, then fall on 16 disjoint groups of 4 banks
  static constexpr int kKRow = D + 8;
  struct Smem : EpilogueSmem<G, D, kWaves> {
    unsigned short vst[kWaves][kBlock * D];     // each wave's staged V block
    unsigned short kst[kWaves][kBlock * kKRow];  // and K block
  };

  const int col, grp;
  const float inv_qk;  // 1 / qk_scale: the raise threshold in raw score units
  Smem* smp = nullptr;
  Vec8<__bf16> qf[KC];  // Q^T fragments: head col (zero past G), dims 32c + 8 grp .. +7
  float mq, thr;        // the head's running max (log2 units) and its raise threshold
  f32x4_t o[NH], ls;    // O^T accumulators; the weight sum in element 0 of the lanes grp == 0

  __device__ __forceinline__ explicit WorkerM(const DecodeArgs& args)
      : Base(args), col(lane & 15), grp(lane >> 4), inv_qk(1.0f / qk_scale) {}

  __device__ __forceinline__ void bind(Smem& sm) { smp = &sm; }

  __device__ __forceinline__ void load_queries(int row, int g) {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (size_t)row * a.q_row_stride +
                       ((size_t)g * G + (col < G ? col : 0)) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (col < G) qf[c].load_cached(qp + 32 * c);
      else qf[c].zero();
    }
  }
  __device__ __forceinline__ void load_queries_from(const __bf16* qs) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (col < G) qf[c].load_cached(qs + col * D + 32 * c + 8 * grp);
      else qf[c].zero();
    }
  }

  // Rotate the queries at pos (pools with RoPE tables; each piece's partner half, dims d ^ D/2,
  // is read from qset, the chunk's G x D queries in memory or in LDS) with the append kernel's
  // arithmetic, and, in split 0, store them to q_out.
  __device__ __forceinline__ void fused_queries(const Chunk& ch, int pos, const __bf16* qset) {
    if (col >= G) return;
    if (a.cos != nullptr) {
#pragma clang fp contract(off)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int d0 = 32 * c + 8 * grp;
        const size_t i0 = (size_t)pos * (D / 2) + (size_t)(d0 & (D / 2 - 1));
        const float4* cp = reinterpret_cast<const float4*>(a.cos + i0);
        const float4* sp = reinterpret_cast<const float4*>(a.sin + i0);
        const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        Vec8<__bf16> other;
        other.load_cached(qset + col * D + (d0 ^ (D / 2)));
        float x[8], y[8], r[8];
        qf[c].to_f32(x);
        other.to_f32(y);
        const bool low = d0 < D / 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = x[e] * cs[e];
          const float p1 = y[e] * sn[e];
          r[e] = low ? p0 - p1 : p0 + p1;
        }
        qf[c].from_f32(r);
      }
    }
    if (a.q_out != nullptr && ch.split == 0 && wave == 0) {
      __bf16* qo = reinterpret_cast<__bf16*>(a.q_out) +
                   ((size_t)ch.row * a.H_q + (size_t)ch.g * G + col) * D + 8 * grp;
#pragma unroll
      for (int c = 0; c < KC; ++c) qf[c].store(qo + 32 * c);
    }
  }

  __device__ __forceinline__ void reset() {
    mq = kNegInf;
    thr = kNegInf;
    ls = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NH; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void load_block(Frag& f, const Chunk& ch, int ids, int blk) const {
    if constexpr (PADDED) {
      const size_t head_base = ((size_t)ch.row * a.H_kv + ch.g) * (size_t)a.seq_cap * D;
      auto column = [&](int key) {
        const int tv = ch.tok0 + blk * kBlock + key;
        const int cc = tv < ch.gap_s ? tv : tv + ch.gap_shift;
        return cc < a.kv_cols ? cc : a.kv_cols - 1;
      };
#pragma unroll
      for (int c = 0; c < VC; ++c) {
        const int e = lane * 8 + 512 * c;  // element of the [16][D] block: key e / D, dim e % D
        const size_t off = head_base + (size_t)column(e / D) * D + e % D;
        f.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kbase + off));
        f.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vbase + off));
      }
    } else {
      const int pb = this->clamp_id(__builtin_amdgcn_readlane(ids, blk));
      const size_t boff = ((size_t)pb * a.H_kv + ch.g) * (size_t)(kBlock * D);
      const char* kb = reinterpret_cast<const char*>(kbase + boff);
      const char* vb = reinterpret_cast<const char*>(vbase + boff);
      // a 32-bit lane offset on a wave-uniform base: the scalar-base form of the global load
      unsigned lo = (unsigned)(lane * 16);
      asm volatile("" : "+v"(lo));
#pragma unroll
      for (int c = 0; c < VC; ++c) {
        f.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + lo + 1024 * c));
        f.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + lo + 1024 * c));
      }
    }
  }

  // One block. MASK is for the chunk's partial last block: its slots past the chunk end may hold
  // anything (NaN included) and never reach the sums.
  template <bool MASK>
  __device__ __forceinline__ void update(const Frag& f, const Chunk& ch, int blk) {
    unsigned short* vst = smp->vst[wave];
    unsigned short* kst = smp->kst[wave];
    u32x4_t* vs = reinterpret_cast<u32x4_t*>(vst);
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      const int e = lane * 8 + 512 * c;
      *reinterpret_cast<u32x4_t*>(kst + (e / D) * kKRow + e % D) = f.k[c];
      vs[lane + 64 * c] = f.v[c];
    }
    __builtin_amdgcn_wave_barrier();
    // K fragments (A operand): key col, dims 32c + 8 grp .. +7
    u32x4_t kf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c)
      kf[c] = *reinterpret_cast<const u32x4_t*>(kst + col * kKRow + 32 * c + 8 * grp);
    const int key0 = blk * kBlock + 4 * grp;
    bool valid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) valid[j] = !MASK || key0 + j < ch.ntok;
    // V^T fragments (dims 16t + col, keys 4 grp .. +3), read now so the LDS latency hides behind
    // the score product
    const unsigned short* vtr = vst + (4 * grp + col / 4) * D + 4 * (col % 4);
    s16x4_t vt[NH];
#pragma unroll
    for (int t = 0; t < NH; ++t) vt[t] = lds_read_tr16(vtr + 16 * t);
    // D <= 64: the same fragments again, for the other half of the K = 32 product's A operand (the
    // address passes through an empty asm, so the compiler emits a second read, not register copies)
    s16x4_t vt2[NH];
    if constexpr (kK32) {
      int vz = 0;
      asm("" : "+v"(vz));
#pragma unroll
      for (int t = 0; t < NH; ++t) vt2[t] = lds_read_tr16(vtr + vz + 16 * t);
    }
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[c]),
                                                  __builtin_bit_cast(bf16x8_t, qf[c].w), s, 0, 0,
                                                  0);
    if (MASK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = valid[j] ? s[j] : kNegInf;
    }
    const float lm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__builtin_amdgcn_ballot_w64(lm > thr) != 0) {
      float bm = fmaxf(lm, swap_rows16(lm));
      bm = fmaxf(bm, swap_halves32(bm));
      const float bms = bm * qk_scale;
      if (bms > mq + kRescale) {
        const float al = exp2_fast(mq - bms);
        ls[0] *= al;  // the other elements hold zero
#pragma unroll
        for (int t = 0; t < NH; ++t) o[t] *= al;
        mq = bms;
        thr = (bms + kRescale) * inv_qk;
      }
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = exp2_fast(fmaf(s[j], qk_scale, -mq));
      if (MASK) p[j] = valid[j] ? p[j] : 0.f;  // a head with only masked keys has mq = -inf
    }
    unsigned h01, h23, l01, l23;
    split_bf16x2(p[0], p[1], h01, l01);
    split_bf16x2(p[2], p[3], h23, l23);
    const s16x4_t p_hi = __builtin_bit_cast(s16x4_t, u32x2_t{h01, h23});
    const s16x4_t p_lo = __builtin_bit_cast(s16x4_t, u32x2_t{l01, l23});
    const short one = col == 0 ? (short)0x3F80 : (short)0;  // bf16 1.0 in row 0 of the A operand
    const s16x4_t ones = {one, one, one, one};
    if constexpr (kK32) {
      // k 0..3 of a lane's group carry the hi weights, k 4..7 the lo weights of the same keys
      const bf16x8_t pb =
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(p_hi, p_lo, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8_t ones8 =
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ones, ones, 0, 1, 2, 3, 0, 1, 2, 3));
      ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb, ls, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        if (MASK) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vt[t][j] = valid[j] ? vt[t][j] : (short)0;
            vt2[t][j] = valid[j] ? vt2[t][j] : (short)0;
          }
        }
        const bf16x8_t va = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(vt[t], vt2[t], 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[t], 0, 0, 0);
      }
    } else {
      ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, p_hi, ls, 0, 0, 0);
      ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, p_lo, ls, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        if (MASK) {
#pragma unroll
          for (int j = 0; j < 4; ++j) vt[t][j] = valid[j] ? vt[t][j] : (short)0;
        }
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[t], p_hi, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[t], p_lo, o[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // A ring of three fragments (two blocks in flight while one is computed), for grids that the
  // device holds at once: a wave then has its SIMD nearly to itself, and with the products on the
  // matrix cores it waits on its loads. Block b sits in the fragment b mod 3; every load in the loop
  // is unconditional (past the wave's last block it re-reads that block), and the chunk's partial
  // last block is updated masked after the loop. The updates run in run_blocks' order: the same
  // bits.
  __device__ __forceinline__ void run_blocks3(Frag& f0, Frag& f1, const Chunk& ch, int ids, int my) {
    Frag f2;
    if (my <= 0) return;
    const int last = my - 1;
    auto clamp = [&](int b) { return this->blk_of(b < last ? b : last); };
    load_block(f1, ch, ids, clamp(1));
    const bool tail = this->blk_of(last) == ch.tail_blk;
    const int steady = tail ? last : my;  // blocks that take the unmasked update
    for (int i = 0; i < steady; i += 3) {
      load_block(f2, ch, ids, clamp(i + 2));
      update<false>(f0, ch, this->blk_of(i));
      load_block(f0, ch, ids, clamp(i + 3));
      if (i + 1 < steady) update<false>(f1, ch, this->blk_of(i + 1));
      load_block(f1, ch, ids, clamp(i + 4));
      if (i + 2 < steady) update<false>(f2, ch, this->blk_of(i + 2));
    }
    if (tail) {
      const int slot = last % 3;
      if (slot == 0) update<true>(f0, ch, this->blk_of(last));
      else if (slot == 1) update<true>(f1, ch, this->blk_of(last));
      else update<true>(f2, ch, this->blk_of(last));
    }
  }

  // Worker::run_blocks' schedule (two fragments swapping roles, the partial last block masked)
  // with this worker's loads and updates.
  __device__ __forceinline__ void run_blocks(Frag& f0, Frag& f1, const Chunk& ch, int ids, int my) {
    int i = 0;
    for (; i + 2 < my; i += 2) {
      load_block(f1, ch, ids, this->blk_of(i + 1));
      update<false>(f0, ch, this->blk_of(i));
      load_block(f0, ch, ids, this->blk_of(i + 2));
      update<false>(f1, ch, this->blk_of(i + 1));
    }
    const bool tail = my > 0 && this->blk_of(my - 1) == ch.tail_blk;
    if (i + 1 < my) {
      load_block(f1, ch, ids, this->blk_of(i + 1));
      update<false>(f0, ch, this->blk_of(i));
      if (tail) update<true>(f1, ch, this->blk_of(i + 1));
      else update<false>(f1, ch, this->blk_of(i + 1));
    } else if (i < my) {
      if (tail) update<true>(f0, ch, this->blk_of(i));
      else update<false>(f0, ch, this->blk_of(i));
    }
  }

  // Park the wave's per-head state in LDS for the combination across waves (then a barrier).
  __device__ __forceinline__ void merge_to_smem(Smem& sm) {
    if (col < G) {
#pragma unroll
      for (int t = 0; t < NH; ++t)
        *reinterpret_cast<f32x4_t*>(&sm.acc[wave][col][16 * t + 4 * grp]) = o[t];
      if (grp == 0) {
        sm.m[wave][col] = mq;
        sm.l[wave][col] = ls[0];
      }
    }
    __syncthreads();
  }
};

// The worker of each element type: bf16 on the matrix cores (PA_DECODE_MFMA = 1), fp32 on the
// vector ALUs.
#ifndef PA_DECODE_MFMA
#define PA_DECODE_MFMA 1
#endif
template <typename T, int D, int G, bool PADDED>
struct DecodeWorker {
  using type = Worker<T, D, G, PADDED>;
};
template <int D, int G, bool PADDED>
struct DecodeWorker<__bf16, D, G, PADDED> {
  using type = std::conditional_t<PA_DECODE_MFMA != 0, WorkerM<D, G, PADDED>,
                                  Worker<__bf16, D, G, PADDED>>;
};

// Valid tokens of a row (and, padded, its gap start and width), lengths clamped to the bounds,
// from the row's loaded values: l0 = gap_start[row] and l1 = gap_end[row] (padded), or l0 =
// kv_lens[row] (positions[row] for a lockstep step; l1 unused).
template <bool PADDED>
__device__ __forceinline__ int row_valid_raw(const DecodeArgs& a, int l0, int l1, int* gap_s,
                                             int* gap_shift) {
  if constexpr (PADDED) {
    const int cols = a.kv_cols;
    const int gs = clampi(l0, 0, cols);
    const int ge = clampi(l1, gs, cols);
    *gap_s = gs;
    *gap_shift = ge - gs;
    return cols - (ge - gs);
  } else {
    *gap_s = 0;
    *gap_shift = 0;
    if (a.kv_from_positions)  // kv_len = position + 1
      return l0 < 0 ? 0 : (l0 >= a.max_kv_len ? a.max_kv_len : l0 + 1);
    return clampi(l0, 0, a.max_kv_len);
  }
}

// The same, loading the row's values.
template <bool PADDED>
__device__ __forceinline__ int row_valid(const DecodeArgs& a, int row, int* gap_s, int* gap_shift) {
  if constexpr (PADDED)
    return row_valid_raw<true>(a, a.gap_start[row], a.gap_end[row], gap_s, gap_shift);
  else
    return row_valid_raw<false>(a, a.kv_from_positions ? a.positions[row] : a.kv_lens[row], 0,
                                gap_s, gap_shift);
}

// Lockstep step: the row's position for the next step, written once per row (by the workgroup of
// KV head 0, split 0, which every row has) to a buffer no workgroup of this launch reads.
__device__ __forceinline__ void advance_position(const DecodeArgs& a, const Chunk& ch) {
  if (a.positions_out != nullptr && ch.g == 0 && ch.split == 0 && threadIdx.x == 0)
    a.positions_out[ch.row] = a.positions[ch.row] + 1;
}

// ---- merge of a row's splits inside the split grid ----------------------------------------------
// In a launch where no row has more than kGridMergeSplits splits, the workgroup that finishes the
// last split of a (row, KV head) -- known from a count of finished splits in the workspace --
// merges the partials of the G query heads, one wave per head. The arithmetic is that of
// lse_reduce_kernel's single-wave merge (which every row of at most 16 splits takes there): the
// same maximum, the weights summed by lane and then across the wave, the outputs accumulated in
// split order. A row therefore gets the same bits whichever of the two merges it.
constexpr int kGridMergeSplits = 16;

// A load that sees device-coherent stores of other workgroups (it does not hit stale lines of this
// XCD's L2).
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__device__ __forceinline__ void merge_splits_one_wave(const DecodeArgs& a, int row, int hq, int ns,
                                                      int lane) {
  const size_t base = ((size_t)row * a.H_q + hq) * a.s_max;
  const float* po = a.part_o + base * D;
  // every split's output in one round of loads (indices clamped to the last split; the extra
  // slots are never summed)
  float v0[kGridMergeSplits], v1[kGridMergeSplits];
#pragma unroll
  for (int i = 0; i < kGridMergeSplits; ++i) {
    const int si = i < ns ? i : ns - 1;
    v0[i] = lane < D ? coherent_load(po + (size_t)si * D + lane) : 0.f;
    v1[i] = D > 64 ? coherent_load(po + (size_t)si * D + 64 + lane) : 0.f;
  }
  const float ls = lane < ns ? coherent_load(a.part_lse + base + lane) : kNegInf;
  float mx = ls;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float w = (ls == kNegInf) ? 0.f : exp2_fast(ls - mx);
  float W = 0.f;
  W += w;
  const int wb = __builtin_bit_cast(int, w);
  float A0 = 0.f, A1 = 0.f;
#pragma unroll
  for (int k = 0; k < kGridMergeSplits; k += 8) {
    if (k < ns) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // lanes past the splits hold w = 0, and their slots add 0 * 0
        const bool ok = k + i < ns;
        const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wb, k + i));
        A0 = fmaf(wk, ok ? v0[k + i] : 0.f, A0);
        A1 = fmaf(wk, ok ? v1[k + i] : 0.f, A1);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  float* out = a.out + ((size_t)row * a.H_q + hq) * D;
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if (lane < D) out[lane] = A0 * inv;
  if (D > 64) out[64 + lane] = A1 * inv;
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)row * a.H_q + hq] = W > 0.f ? (mx + __log2f(W)) * kLn2 : kNegInf;
}

// Waves that merge one row's splits: a function of the row's own split count only, so a row's
// result never depends on the rest of the batch. lse_reduce_kernel brings reduce_waves(s_max) waves
// per (row, query head).
__host__ __device__ constexpr int reduce_waves(int ns) { return ns <= 16 ? 1 : (ns <= 64 ? 4 : 8); }
// Splits per merging wave: a row of at most 16 splits is merged by one wave; up to 64, by waves of
// 16 consecutive splits; up to 256, of 32; beyond, ceil(ns / 8) each. A function of the row's own
// split count, so a row's merge is the same in any batch, and fixed over wide ranges of it, so the
// waves can load their ranges before the row length arrives.
__host__ __device__ constexpr int split_range(int ns) {
  return ns <= 16 ? 16 : (ns <= 64 ? 16 : (ns <= 256 ? 32 : (ns + 7) / 8));
}
// partial outputs per batch of loads of a wave's range
template <int NW>
constexpr int merge_batch() { return NW == 1 ? 8 : (NW == 4 ? 16 : 32); }

// Called by every thread of a workgroup whose chunk wrote its partial result with device-coherent
// stores. No cache-wide fence is taken (an L2 write-back and invalidate per workgroup would stall
// the whole launch): each thread waits for its own stores to be acknowledged, the workgroup meets
// at a barrier, and only then is the count bumped; the merging wave reads with device-coherent
// loads. (Rows of more than 16 splits are left to lse_reduce_kernel: a two-level merge of their
// ranges inside the grid, by the last workgroup of each range and then of the row, gave the
// kernel's bits but lengthened the end of the launch, 185.0 against 184.7 us on the long-context
// step and 56.3 against 50.3 us on one GPU's quarter of it.)
template <int D, int G>
__device__ __forceinline__ void merge_if_last(const DecodeArgs& a, const Chunk& ch, int lane,
                                              int wave, int* s_last) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* cnt = a.merge_counts + (size_t)ch.row * a.H_kv + ch.g;
  if (threadIdx.x == 0)
    *s_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      ch.ns - 1
                  ? 1
                  : 0;
  __syncthreads();
  if (*s_last == 0) return;
  if (threadIdx.x == 0)  // re-armed for the next call
    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int h = wave; h < G; h += kWaves)
    merge_splits_one_wave<D>(a, ch.row, ch.g * G + h, ch.ns, lane);
}

// ---- grid kernel: one workgroup per (KV head, row, split); splits past the row's end exit -------
// COMPACT (batches of at most 64 rows): a 1-D grid whose workgroups map to the chunks through
// the rows' lengths, every row's full chunks first and each row's partial last chunk after them,
// so the workgroups past the last chunk (which exit at once) all come at the end of the launch.
// Workgroups per CU the bf16 grid kernels are compiled for: 3 caps them at 168 VGPRs, 3 waves per
// SIMD. The D = 128 instances would otherwise take 169 and run 2 waves per SIMD; held to 168 the
// long-context decode (compact grid) is 0.4 us faster, with no spills. 0 leaves the register
// budget to the compiler.
#ifndef PA_DECODE_MIN_WG_PER_CU
#define PA_DECODE_MIN_WG_PER_CU 3
#endif
template <typename T, int G>
constexpr int grid_min_wg() {
  // G = 8 instances need more registers than 3 waves per SIMD allow: they would spill
  return sizeof(T) == 2 && G <= 4 && PA_DECODE_MIN_WG_PER_CU > 0 ? PA_DECODE_MIN_WG_PER_CU : 1;
}

// Ticket of a workgroup of the ticketed split grid (the workgroups of grid rows >= ticket_y): the
// count of such workgroups that asked before it. The counter (bytes 8-15 of the workspace) holds
// the tickets handed out in its low half and the workgroups that asked in its high half; every
// ticketed workgroup asks exactly once, so the last to ask re-arms it to zero for the next call.
// An XCD that runs ahead starts its ticketed workgroups sooner and so takes more of the last
// chunks; the ticketed workgroups left on a slower XCD find none and exit.
__device__ __forceinline__ int take_ticket(const DecodeArgs& a) {
  __shared__ int s_ticket;
  if (threadIdx.x == 0) {
    unsigned long long* ctr = reinterpret_cast<unsigned long long*>(a.counter) + 1;
    const unsigned long long old = __hip_atomic_fetch_add(
        ctr, (1ull << 32) | 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned asking = (gridDim.y - (unsigned)a.ticket_y) * gridDim.x;
    if ((unsigned)(old >> 32) == asking - 1)
      __hip_atomic_store(ctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ticket = (int)(unsigned)old;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_ticket);
}

// RING = 3: the bf16 worker's three-fragment ring (run_blocks3), for split grids the device holds
// at once.
template <typename T, int D, int G, bool PADDED, bool COMPACT, int RING = 2>
__global__ __launch_bounds__(64 * kWaves, (grid_min_wg<T, G>())) void decode_vector_kernel(
    const DecodeArgs a) {
  using W = typename DecodeWorker<T, D, G, PADDED>::type;
  __shared__ typename W::Smem sm;
  W w(a);
  w.bind(sm);
  const int chunk = chunk_tokens(D);
  int g, row, split;
  int n = 0, gap_s = 0, gap_shift = 0;
  if constexpr (COMPACT) {
    // one row per lane: its valid tokens, its full chunks and whether it has a partial one
    int gs_l = 0, gsh_l = 0;
    const bool has = w.lane < a.batch;
    const int nb = has ? row_valid<PADDED>(a, w.lane, &gs_l, &gsh_l) : 0;
    int f = 0, pc = 0;
    if (has) chunk_groups(nb, chunk, &f, &pc);
    int fi = f, pi = pc;  // inclusive prefix sums over the rows
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int fu = __shfl_up(fi, o), pu = __shfl_up(pi, o);
      if (w.lane >= o) {
        fi += fu;
        pi += pu;
      }
    }
    const int n_full = __builtin_amdgcn_readlane(fi, 63);
    const int n_part = __builtin_amdgcn_readlane(pi, 63);
    const int item = (int)(blockIdx.x / (unsigned)a.H_kv);
    g = (int)(blockIdx.x % (unsigned)a.H_kv);
    if (item >= n_full + n_part) return;  // past the last chunk: these come last
    const bool full = item < n_full;
    const int k = full ? item : item - n_full;
    // the one row whose range holds k (rows with an empty range never match)
    const unsigned long long m =
        full ? __ballot(has && fi - f <= k && k < fi) : __ballot(has && pi - pc <= k && k < pi);
    if (m == 0) return;  // cannot happen: the rows' ranges cover every item
    row = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(m));
    n = __builtin_amdgcn_readlane(nb, row);
    gap_s = __builtin_amdgcn_readlane(gs_l, row);
    gap_shift = __builtin_amdgcn_readlane(gsh_l, row);
    split = full ? k - (__builtin_amdgcn_readlane(fi, row) - __builtin_amdgcn_readlane(f, row))
                 : n / chunk;
  } else if (a.ticket_y == 0) {
    g = blockIdx.x;
    row = blockIdx.y;
    // the highest splits go first: they exist only for the longest rows, so the launch ends with
    // the splits every row has (a shorter drain than ending on long rows' late full chunks)
    split = (int)gridDim.z - 1 - (int)blockIdx.z;
  } else {
    // ticketed grid: grid rows y < ticket_y hold the same fixed chunks, in the same order, as the
    // plain grid's (y = row + batch * (s_max - 1 - split)); past them, each workgroup takes the
    // next of the remaining split-0 chunks from a counter, or exits when none is left
    const int y = (int)blockIdx.y;
    if (y < a.ticket_y) {
      g = blockIdx.x;
      row = y % a.batch;
      split = a.s_max - 1 - y / a.batch;
    } else {
      const int c = take_ticket(a) + (a.ticket_y - a.batch * (a.s_max - 1)) * a.H_kv;
      if (c >= a.batch * a.H_kv) return;
      row = c / a.H_kv;
      g = c - row * a.H_kv;
      split = 0;
    }
  }
  // issued before the row length is known, so their latency overlaps the length load
  int ids = w.load_ids(row, split * chunk);
  w.load_queries(row, g);
  // The row's scalars: its length (or gap) and, for the fused append, its position (a table row,
  // clamped) for the rotations and where its new token goes. They are loaded together, with no
  // branch between the loads (one a call does not need re-reads the length), so one wait covers
  // them; behind a branch, each had waited for every load issued before it.
  const bool fused = a.k_new != nullptr;
  const int32_t* lp = PADDED ? a.gap_start : (a.kv_from_positions ? a.positions : a.kv_lens);
  const int32_t* ep = PADDED ? a.gap_end : lp;
  const int32_t* tp = fused ? (a.dest != nullptr ? a.dest : a.positions) : lp;
  const int32_t* pp = fused && a.cos != nullptr ? a.positions : lp;
  // The pointers are opaque to the compiler, which would otherwise turn a load it can prove equal
  // to another back into a branch around a load; the four values then pass through one empty asm
  // before any is used, so they are loaded together (left to itself, the compiler waits for the
  // length alone, for the early exit below, and issues the others after it: a second round trip)
  asm("" : "+s"(lp), "+s"(ep), "+s"(tp), "+s"(pp));
  typedef const __attribute__((address_space(1))) int32_t gint;
  int v_l0 = ((gint*)lp)[row], v_l1 = ((gint*)ep)[row];
  int v_t = ((gint*)tp)[row], v_p = ((gint*)pp)[row];
  asm volatile("" : "+v"(v_l0), "+v"(v_l1), "+v"(v_t), "+v"(v_p));
  const int l0 = __builtin_amdgcn_readfirstlane(v_l0);
  const int l1 = __builtin_amdgcn_readfirstlane(v_l1);
  const int t_raw = __builtin_amdgcn_readfirstlane(v_t);
  const int p_raw = __builtin_amdgcn_readfirstlane(v_p);
  const int pos = fused && a.cos != nullptr ? clampi(p_raw, 0, a.rope_max_pos - 1) : 0;
  const int t_new = fused ? w.fused_clamp(t_raw) : 0;
  Vec8<T> kx, kp, vx;
  if constexpr (!COMPACT) n = row_valid_raw<PADDED>(a, l0, l1, &gap_s, &gap_shift);
  const Chunk ch = make_chunk(row, g, split, n, gap_s, gap_shift, chunk);
  if (split >= ch.ns) return;
  advance_position(a, ch);
  bool first = false;
  const bool stores = fused && w.fused_target(ch, n, t_new, &first);
  // only the wave that stores the token loads its pieces of the new key and value (loaded by every
  // workgroup up front, they cost the fused step 0.4-3.6 us on B=128)
  if (stores && w.lane < W::LPT) w.fused_load(row, g, kx, kp, vx);
  if (stores && first) {
    // the token's block is the next load of this wave: its stores complete first
    w.fused_store(kx, kp, vx, ch, t_new, pos);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  w.reset();
  typename W::Frag f0, f1;
  const int my = w.my_blocks(ch);
  if (my > 0) w.load_block(f0, ch, ids, w.blk_of(0));
  if (stores && !first) w.fused_store(kx, kp, vx, ch, t_new, pos);
  if (fused)  // while the first block is in flight
    w.fused_queries(ch, pos, reinterpret_cast<const T*>(a.q) + (size_t)row * a.q_row_stride +
                                 (size_t)g * G * D);
  if constexpr (RING == 3) w.run_blocks3(f0, f1, ch, ids, my);
  else w.run_blocks(f0, f1, ch, ids, my);
  w.merge_to_smem(sm);
  w.write_result(sm, ch);
  if constexpr (!COMPACT) {
    // merge_counts is set only for the split grid, when no row of the launch has more than
    // kGridMergeSplits splits (the compact grid leaves the merge to lse_reduce_kernel: carrying
    // the unused merge code made its long-context launch 1.7 us slower)
    if (a.merge_counts != nullptr && ch.ns > 1) {
      __shared__ int s_last;
      merge_if_last<D, G>(a, ch, w.lane, w.wave, &s_last);
    }
  }
}

// ---- persistent kernel --------------------------------------------------------------------------
// A fixed grid of workgroups (as many as fit on the device) takes chunks (after two fixed ones
// each) from a counter in the workspace, in an order that puts every row's full chunks first and
// the shorter last chunks at the end, so no workgroup slot is spent on a split past a row's end. A workgroup knows its next chunk
// one step ahead: while the current chunk streams, that chunk's block ids and queries are loaded
// and parked in LDS, and its first K/V block is in flight while the current chunk's result is
// merged and written. The split of each row is the same
// as in the grid kernel, so results are identical.
constexpr int kMaxRows = 1024;
constexpr int kPersistentMinSplits = 16;  // s_max from which the persistent launch is used

template <bool PADDED>
struct RowSmem {
  int n[kMaxRows];
  int full_pre[kMaxRows + 1];  // exclusive prefix over rows of full chunks (n / chunk)
  int part_pre[kMaxRows + 1];  // exclusive prefix over rows of last partial chunks (0 or 1)
  int gap_s[PADDED ? kMaxRows : 1];
  int gap_shift[PADDED ? kMaxRows : 1];
  int wave_tot[2][kWaves];
  int ticket[3];
};

// Exclusive prefix sums over rows of (full, partial) chunk counts into LDS; rows are split into
// contiguous runs per thread, then a two-level scan over threads.
template <bool PADDED>
__device__ void scan_rows(RowSmem<PADDED>& rs, int B, int chunk) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kPer = (kMaxRows + kThreads - 1) / kThreads;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int fl[kPer], pl[kPer];
  int fs = 0, ps = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = t * kPer + i;
    int f = 0, p = 0;
    if (b < B) chunk_groups(rs.n[b], chunk, &f, &p);
    fl[i] = fs;
    pl[i] = ps;
    fs += f;
    ps += p;
  }
  // inclusive scan of the per-thread totals within the wave
  int fi = fs, pi = ps;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int fu = __shfl_up(fi, o);
    const int pu = __shfl_up(pi, o);
    if (lane >= o) {
      fi += fu;
      pi += pu;
    }
  }
  if (lane == 63) {
    rs.wave_tot[0][wave] = fi;
    rs.wave_tot[1][wave] = pi;
  }
  __syncthreads();
  int fw = 0, pw = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    fw += rs.wave_tot[0][w2];
    pw += rs.wave_tot[1][w2];
  }
  const int fbase = fw + fi - fs, pbase = pw + pi - ps;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = t * kPer + i;
    if (b < B) {
      rs.full_pre[b] = fbase + fl[i];
      rs.part_pre[b] = pbase + pl[i];
    }
  }
  if (t == 0) {
    int ft = 0, pt = 0;
    for (int w2 = 0; w2 < kWaves; ++w2) {
      ft += rs.wave_tot[0][w2];
      pt += rs.wave_tot[1][w2];
    }
    rs.full_pre[B] = ft;
    rs.part_pre[B] = pt;
  }
  __syncthreads();
}

// LDS reads land in vector registers; every workgroup-uniform value read from LDS goes through
// readfirstlane so that the compiler keeps it (and all that derives from it) scalar.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ Chunk uni_chunk(const Chunk& c) {
  Chunk u;
  u.row = uni(c.row);
  u.g = uni(c.g);
  u.split = uni(c.split);
  u.tok0 = uni(c.tok0);
  u.ntok = uni(c.ntok);
  u.nblk = uni(c.nblk);
  u.tail_blk = uni(c.tail_blk);
  u.ns = uni(c.ns);
  u.gap_s = uni(c.gap_s);
  u.gap_shift = uni(c.gap_shift);
  return u;
}

// last index b in [0, B) with pre[b] <= k (pre non-decreasing, pre[B] > k)
__device__ __forceinline__ int find_row(const int* pre, int B, int k) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(pre[mid]) <= k) lo = mid; else hi = mid;
  }
  return lo;
}

template <bool PADDED>
__device__ __forceinline__ Chunk decode_ticket(const RowSmem<PADDED>& rs, int B, int H_kv,
                                               int n_full, int t, int chunk) {
  int k = t / H_kv;
  const int g = t - k * H_kv;
  int row, split;
  if (k < n_full) {
    row = find_row(rs.full_pre, B, k);
    split = k - rs.full_pre[row];
  } else {
    k -= n_full;
    row = find_row(rs.part_pre, B, k);
    split = rs.n[row] / chunk;
  }
  const int gs = PADDED ? uni(rs.gap_s[row]) : 0;
  const int gsh = PADDED ? uni(rs.gap_shift[row]) : 0;
  return make_chunk(uni(row), uni(g), uni(split), uni(rs.n[row]), gs, gsh, chunk);
}

template <typename T, int D, int G, bool PADDED>
__global__ __launch_bounds__(64 * kWaves) void decode_persistent_kernel(
    const DecodeArgs a) {
  using W = typename DecodeWorker<T, D, G, PADDED>::type;
  constexpr int kQVec = G * D * (int)sizeof(T) / 16;  // 16-byte pieces of one (row, g) query set
  static_assert(kQVec <= 64 * kWaves, "query staging: at most one piece per thread");
  __shared__ typename W::Smem sm;
  __shared__ RowSmem<PADDED> rs;
  __shared__ int s_ids[2][64];
  __shared__ uint4 s_q[2][kQVec];
  W w(a);
  w.bind(sm);
  const int B = a.batch;
  const int chunk = chunk_tokens(D);
  int* counter = a.counter;
  const int tid = threadIdx.x;

  // The first two chunks of every workgroup are fixed by its index; later ones come from the
  // counter, offset past them (so the launch does not start with every workgroup contending for
  // one atomic).
  const int n_static = 2 * (int)gridDim.x;
  for (int b = tid; b < B; b += 64 * kWaves) {
    int gs, gsh;
    rs.n[b] = row_valid<PADDED>(a, b, &gs, &gsh);
    if constexpr (PADDED) {
      rs.gap_s[b] = gs;
      rs.gap_shift[b] = gsh;
    }
  }
  __syncthreads();
  scan_rows<PADDED>(rs, B, chunk);
  const int n_full = uni(rs.full_pre[B]);
  const int n_items = (n_full + uni(rs.part_pre[B])) * a.H_kv;

  int t_cur = (int)blockIdx.x;
  int t_nxt = (int)(blockIdx.x + gridDim.x);
  if (t_cur >= n_items) return;  // uniform: no work left for this workgroup

  // a chunk's block ids (wave 0) and queries (one 16-byte piece per thread): global -> registers,
  // later parked in LDS
  auto fetch = [&](const Chunk& ch, int& pid, uint4& pq) {
    if (w.wave == 0) pid = w.load_ids(ch.row, ch.tok0);
    if (tid < kQVec) {
      const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)ch.row * a.q_row_stride +
                    (size_t)ch.g * G * D;
      pq = reinterpret_cast<const uint4*>(qp)[tid];
    }
  };
  auto park = [&](int slot, int pid, const uint4& pq) {
    if (w.wave == 0) s_ids[slot][w.lane] = pid;
    if (tid < kQVec) s_q[slot][tid] = pq;
  };

  // fused append: store a chunk's new token and wait for the stores (its block is this wave's
  // next load)
  const bool fused = a.k_new != nullptr;
  auto store_now = [&](const Chunk& ch, int t, int p) {
    Vec8<T> kx, kp, vx;
    if (w.lane < W::LPT) w.fused_load(ch.row, ch.g, kx, kp, vx);
    w.fused_store(kx, kp, vx, ch, t, p);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  Chunk cur = decode_ticket<PADDED>(rs, B, a.H_kv, n_full, t_cur, chunk);
  {
    int pid = 0;
    uint4 pq = make_uint4(0, 0, 0, 0);
    fetch(cur, pid, pq);
    park(0, pid, pq);
  }
  __syncthreads();
  bool has_nx = t_nxt < n_items;
  typename W::Frag f0, f1;
  bool pre = false;  // f0 already holds (in flight) this wave's first block of `cur`
  for (int k = 0;; ++k) {
    const int slot = k & 1;
    // the chunk after next: its ticket is read after this chunk's merge barrier
    if (tid == 0 && has_nx) rs.ticket[(k + 2) % 3] = n_static + atomicAdd(counter, 1);
    const int ids = s_ids[slot][w.lane];
    const T* qs = reinterpret_cast<const T*>(s_q[slot]);
    w.load_queries_from(qs);
    Chunk nx = cur;
    int pid = 0;
    uint4 pq = make_uint4(0, 0, 0, 0);
    if (has_nx) {
      nx = decode_ticket<PADDED>(rs, B, a.H_kv, n_full, t_nxt, chunk);
      fetch(nx, pid, pq);
    }
    // fused append: this chunk's part. A token in this wave's first block (never prefetched, see
    // below) is stored before that block's load, any other one right after the first load.
    int pos = 0, t_new = 0;
    bool stores = false, first = false;
    if (fused) {
      pos = a.cos != nullptr ? clampi(a.positions[cur.row], 0, a.rope_max_pos - 1) : 0;
      t_new = w.fused_index(cur.row);
      stores = w.fused_target(cur, uni(rs.n[cur.row]), t_new, &first);
      if (stores && first) store_now(cur, t_new, pos);
    }
    advance_position(a, cur);
    w.reset();
    const int my = w.my_blocks(cur);
    if (!pre && my > 0) w.load_block(f0, cur, ids, w.blk_of(0));
    if (fused) {
      if (stores && !first) {
        Vec8<T> kx, kp, vx;
        if (w.lane < W::LPT) w.fused_load(cur.row, cur.g, kx, kp, vx);
        w.fused_store(kx, kp, vx, cur, t_new, pos);
      }
      w.fused_queries(cur, pos, qs);
    }
    w.run_blocks(f0, f1, cur, ids, my);
    if (has_nx) park(slot ^ 1, pid, pq);
    w.merge_to_smem(sm);
    // the merge barrier has published the next chunk's block ids: its first block goes in flight
    // before this chunk's results are combined and written
    pre = false;
    if (has_nx) {
      const Chunk nu = uni_chunk(nx);
      // a wave that stores the next chunk's new token into its own first block skips this
      // prefetch: it stores that token at the chunk's start, then loads the block
      bool hold = false;
      if (fused) {
        bool first_nu = false;
        hold = w.fused_target(nu, uni(rs.n[nu.row]), w.fused_index(nu.row), &first_nu) &&
               first_nu;
      }
      if (w.my_blocks(nu) > 0 && !hold) {
        w.load_block(f0, nu, s_ids[slot ^ 1][w.lane], w.blk_of(0));
        pre = true;
      }
    }
    const int t_nn = has_nx ? uni(rs.ticket[(k + 2) % 3]) : n_items;
    w.write_result(sm, cur);
    __syncthreads();  // the merge area and this slot are reused
    if (!has_nx) break;
    cur = uni_chunk(nx);
    t_nxt = t_nn;
    has_nx = t_nxt < n_items;
  }
}


// Merge the split partials of one (row, query head): out = sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - max lse); lse = max + log2(sum w_s), returned in natural-log units.
// Waves share the row's splits in contiguous ranges of split_range(ns); each merges its range
// against its own maximum and wave 0 combines their results in wave order. It is latency-bound,
// so the chain of dependent loads is kept short: every wave's first 64 partial lse values and first
// kSpec partial outputs load together with the row length (speculatively: the workspace always
// holds s_max of each; slots past the range are dropped by a select, so whatever they hold never
// reaches the sums), and later partial outputs load in batches of kSpec (8, 16 or 32 with the
// wave count).
template <bool PADDED, int NW>
__global__ __launch_bounds__(64 * NW) void lse_reduce_kernel(const DecodeArgs a) {
  // partial outputs per batch of loads: a long row's wave covers its whole range in one or two
  constexpr int kSpec = merge_batch<NW>();
  __shared__ float s_acc[NW][128];
  __shared__ float s_mw[NW][2];
  const int hq = blockIdx.x;
  const int row = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = a.D;
  // the decode kernel has finished: re-arm its work counter for the next call
  if (a.counter != nullptr && hq == 0 && row == 0 && threadIdx.x == 0) *a.counter = 0;
  const size_t base = ((size_t)row * a.H_q + hq) * a.s_max;
  const float* po = a.part_o + base * D;
  // this lane's dims (lane, and 64 + lane when D = 128) of the partial outputs of splits
  // s0 + [0, kSpec), indices clamped into [0, last]
  auto load_batch = [&](int s0, int last, float* v0, float* v1) {
#pragma unroll
    for (int i = 0; i < kSpec; ++i) {
      const int si = s0 + i < last ? s0 + i : last;
      const float* p = po + (size_t)si * D;
      v0[i] = lane < D ? p[lane] : 0.f;
      v1[i] = D > 64 ? p[64 + lane] : 0.f;
    }
  };
  // Every wave loads its range before the row length is known: the range of a row's splits per
  // wave is split_range(ns), guessed here as that of the launch's own wave count (exact for every
  // row whose split count takes this many waves, which is the longest ones), and loaded again
  // after the length only when the guess was wrong.
  float v0[kSpec], v1[kSpec];
  const int sb_guess = wave * (NW == 1 ? kSpec : split_range(NW == 4 ? 64 : 256));
  float lse0 = kNegInf;
  if (sb_guess < a.s_max) {
    lse0 = lane < a.s_max - sb_guess ? a.part_lse[base + sb_guess + lane] : kNegInf;
    load_batch(sb_guess, a.s_max - 1, v0, v1);
  }
  int gs, gsh;
  const int n = row_valid<PADDED>(a, row, &gs, &gsh);
  const int ns = num_splits(n, chunk_tokens(D));
  if (ns <= 1) return;  // the same for every wave of the workgroup
  const int per = split_range(ns);
  const int nw = (ns + per - 1) / per;
  const int sb = wave < nw ? wave * per : ns;
  const int se = sb + per < ns ? sb + per : ns;
  if (sb < se && sb != sb_guess) {
    lse0 = lane < se - sb ? a.part_lse[base + sb + lane] : kNegInf;
    load_batch(sb, se - 1, v0, v1);
  }

  float mx = kNegInf, W = 0.f, A0 = 0.f, A1 = 0.f;
  if (sb < se) {
    // maximum over this wave's splits' lse
    mx = lane < se - sb ? lse0 : kNegInf;
    for (int s = sb + 64 + lane; s < se; s += 64) mx = fmaxf(mx, a.part_lse[base + s]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    for (int s0 = sb; s0 < se; s0 += 64) {
      float ls = s0 == sb ? lse0 : (s0 + lane < se ? a.part_lse[base + s0 + lane] : kNegInf);
      if (s0 + lane >= se) ls = kNegInf;
      const float w = (ls == kNegInf) ? 0.f : exp2_fast(ls - mx);
      W += w;
      const int wb = __builtin_bit_cast(int, w);
      const int cnt = se - s0 < 64 ? se - s0 : 64;
      for (int k = 0; k < cnt; k += kSpec) {
        if (s0 + k > sb) load_batch(s0 + k, se - 1, v0, v1);
#pragma unroll
        for (int i = 0; i < kSpec; ++i) {
          const bool ok = k + i < cnt;
          // lanes past the range hold w = 0; the select also drops stale slots' values
          const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wb, (k + i) & 63));
          A0 = fmaf(wk, ok ? v0[i] : 0.f, A0);
          A1 = fmaf(wk, ok ? v1[i] : 0.f, A1);
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  }
  if constexpr (NW > 1) {
    if (lane < D) s_acc[wave][lane] = A0;
    if (D > 64) s_acc[wave][64 + lane] = A1;
    if (lane == 0) {
      s_mw[wave][0] = mx;
      s_mw[wave][1] = W;
    }
    __syncthreads();
    if (wave != 0) return;
    if (nw > 1) {
      float M = kNegInf;
      for (int w = 0; w < nw; ++w) M = fmaxf(M, s_mw[w][0]);
      float Wt = 0.f, B0 = 0.f, B1 = 0.f;
      for (int w = 0; w < nw; ++w) {
        const float mw = s_mw[w][0];
        const float f = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
        Wt = fmaf(f, s_mw[w][1], Wt);
        if (lane < D) B0 = fmaf(f, s_acc[w][lane], B0);
        if (D > 64) B1 = fmaf(f, s_acc[w][64 + lane], B1);
      }
      mx = M;
      W = Wt;
      A0 = B0;
      A1 = B1;
    }
  }
  float* out = a.out + ((size_t)row * a.H_q + hq) * D;
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if (lane < D) out[lane] = A0 * inv;
  if (D > 64) out[64 + lane] = A1 * inv;
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)row * a.H_q + hq] = W > 0.f ? (mx + __log2f(W)) * kLn2 : kNegInf;
}

// Workgroups of `kernel` that fit on the current device at once (per-CU occupancy x CUs), cached
// per (device, kernel, dynamic LDS size).
int resident_workgroups(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(dev, kernel, lds);
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWaves, lds) !=
      hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cache[key] = per_cu * cus;
  return per_cu * cus;
}

// Workgroups of the bf16 split grid per CU. The matrix-core worker's registers would allow 4, and 4
// streaming workgroups per CU measured 1.3% slower than 3 on the B=128 step (more concurrent
// streams for the same bytes): the launch reserves enough unused LDS to hold residency at this.
#ifndef PA_DECODE_GRID_WG_PER_CU
#define PA_DECODE_GRID_WG_PER_CU 3
#endif

// Dynamic LDS that holds `kernel` to at most `per_cu` resident workgroups per CU (0: none needed),
// cached per (device, kernel).
size_t lds_reservation(const void* kernel, int per_cu) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> cache;
  int dev = 0;
  if (per_cu <= 0 || hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_pair(dev, kernel);
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  hipFuncAttributes attr;
  int lds_cu = 0, lds_block = 0;
  size_t pad = 0;
  if (hipFuncGetAttributes(&attr, kernel) == hipSuccess &&
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
          hipSuccess &&
      hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
          hipSuccess &&
      lds_cu > 0) {
    const size_t want = (size_t)lds_cu / (size_t)(per_cu + 1) + 1;  // per_cu + 1 no longer fit
    const size_t own = attr.sharedSizeBytes;
    if (want > own && want <= (size_t)lds_block) pad = (want - own + 255) & ~(size_t)255;
    if (own + pad > (size_t)lds_block) pad = 0;
  }
  cache[key] = pad;
  return pad;
}

// Whether launch_decode_vector takes the persistent kernel for these arguments.
bool decode_vector_is_persistent(const DecodeArgs& a) {
  if (!(PA_DECODE_PERSISTENT && a.counter != nullptr && a.s_max > 1 && a.batch <= kMaxRows))
    return false;
  return PA_DECODE_PERSISTENT == 2 || a.s_max >= kPersistentMinSplits;
}

template <typename T, int D, int G, bool PADDED>
hipError_t launch_layout(const DecodeArgs& args, hipStream_t stream, bool* merged) {
  // only the split grid merges its own splits (and only for rows of at most kGridMergeSplits)
  DecodeArgs a = args;
  a.merge_counts = nullptr;
  *merged = false;
  const long long items = (long long)a.batch * a.H_kv * a.s_max;
  // Rows long enough for many splits: the split grid would cover s_max splits of every row, and
  // the rows' differing lengths leave many of its workgroups with nothing to do, so the persistent
  // kernel takes over. With few splits per row the split grid starts faster (a workgroup needs
  // no row scan before its first loads) and runs more waves per SIMD. Both cut rows into the
  // same chunks: their results are identical.
  if (PA_DECODE_COMPACT && decode_vector_is_persistent(a) && a.batch <= 64 &&
      items <= (long long)0x7fffffff) {
    // Rows with many chunks and few enough rows for one wave to map workgroups to chunks: a
    // compact grid at the split kernel's occupancy (3 waves per SIMD against the persistent
    // kernel's 2), with no early-exit workgroups ahead of working ones. It takes 176-178 us on
    // the B=4 long-context step where the persistent kernel takes 184 us. For short rows the
    // plain grid stays faster: its exits are few and its loads start before the row is known.
    hipLaunchKernelGGL((decode_vector_kernel<T, D, G, PADDED, true>), dim3((unsigned)items),
                       dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
  }
  // fp32 at D = 128, G = 8: the persistent kernel's chunk loop does not fit in 256 registers and
  // would spill (80-104 bytes per lane), so that instance is not built and its rows take the split
  // grid below, which cuts the same chunks
  if constexpr (!(sizeof(T) == 4 && D == 128 && G == 8)) {
    if (decode_vector_is_persistent(a)) {
      auto kern = decode_persistent_kernel<T, D, G, PADDED>;
      const int resident = resident_workgroups(reinterpret_cast<const void*>(kern), 0);
      if (resident > 0 && (PA_DECODE_PERSISTENT == 2 || a.s_max >= kPersistentMinSplits)) {
        const int grid = (int)(items < resident ? items : resident);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWaves), 0, stream, a);
        return hipGetLastError();
      }
    }
  }
  if (PA_DECODE_GRID_MERGE && args.merge_counts != nullptr && a.s_max > 1 &&
      a.s_max <= kGridMergeSplits) {
    a.merge_counts = args.merge_counts;
    *merged = true;
  }
  dim3 grid(a.H_kv, a.batch, a.s_max);
  if constexpr (sizeof(T) == 2 && PA_DECODE_MFMA != 0) {
    auto kern = decode_vector_kernel<T, D, G, PADDED, false>;
    const size_t pad =
        lds_reservation(reinterpret_cast<const void*>(kern), PA_DECODE_GRID_WG_PER_CU);
    // a grid the device holds at once (the lockstep batches) keeps two blocks in flight per wave;
    // not at D = 128, where the third fragment would spill under the 3-waves-per-SIMD register cap
    // (a 16-row batch took 40.6 us spilled against 18.9 us with the two-fragment loop)
    auto ring = decode_vector_kernel<T, D, G, PADDED, false, D <= 64 ? 3 : 2>;
    const size_t ring_pad =
        lds_reservation(reinterpret_cast<const void*>(ring), PA_DECODE_GRID_WG_PER_CU);
    const int resident = resident_workgroups(reinterpret_cast<const void*>(ring), ring_pad);
    if (resident > 0 && items <= resident) {
      hipLaunchKernelGGL(ring, grid, dim3(64 * kWaves), ring_pad, stream, a);
      return hipGetLastError();
    }
    // A grid larger than the device holds ends with a drain whose length differs between the
    // XCDs (each runs the workgroups the dispatcher hands it in turn). The last 3/8 of the split-0
    // chunks are therefore handed out by tickets, to kTicketExtraRows more grid rows than they
    // need: an XCD that runs ahead takes more of them. Same chunks, same bits.
    const long long rows = (long long)a.batch * a.s_max + kTicketExtraRows;
    if (PA_DECODE_TICKETS && a.s_max > 1 && a.counter != nullptr && rows <= 65535) {
      a.ticket_y = a.batch * (a.s_max - 1) + a.batch * 5 / 8;
      hipLaunchKernelGGL(kern, dim3(a.H_kv, (unsigned)rows), dim3(64 * kWaves), pad, stream, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * kWaves), pad, stream, a);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((decode_vector_kernel<T, D, G, PADDED, false>), grid, dim3(64 * kWaves),
                       0, stream, a);
    return hipGetLastError();
  }
}

template <typename T, int D, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream, bool* merged) {
  return a.layout == PA_PADDED ? launch_layout<T, D, G, true>(a, stream, merged)
                               : launch_layout<T, D, G, false>(a, stream, merged);
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream, bool* merged) {
  switch (a.H_q / a.H_kv) {
    case 1: return launch_typed<T, D, 1>(a, stream, merged);
    case 2: return launch_typed<T, D, 2>(a, stream, merged);
    case 4: return launch_typed<T, D, 4>(a, stream, merged);
    case 8: return launch_typed<T, D, 8>(a, stream, merged);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream, bool* merged) {
  switch (a.D) {
    case 32: return launch_d<T, 32>(a, stream, merged);
    case 64: return launch_d<T, 64>(a, stream, merged);
    case 128: return launch_d<T, 128>(a, stream, merged);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_vector(const DecodeArgs& a, hipStream_t stream, bool* merged) {
  *merged = false;
  return a.dtype == PA_F32 ? launch_t<float>(a, stream, merged)
                           : launch_t<__bf16>(a, stream, merged);
}

template <bool PADDED>
hipError_t launch_lse_reduce_layout(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.H_q * a.n_q, a.batch);
  switch (reduce_waves(a.s_max)) {
    case 1:
      hipLaunchKernelGGL((lse_reduce_kernel<PADDED, 1>), grid, dim3(64), 0, stream, a);
      break;
    case 4:
      hipLaunchKernelGGL((lse_reduce_kernel<PADDED, 4>), grid, dim3(256), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((lse_reduce_kernel<PADDED, 8>), grid, dim3(512), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream) {
  return a.layout == PA_PADDED ? launch_lse_reduce_layout<true>(a, stream)
                               : launch_lse_reduce_layout<false>(a, stream);
}

}  // namespace pa
