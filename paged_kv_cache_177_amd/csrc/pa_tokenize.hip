// Fused spike tokenizer + K/V projection into the paged pool, for gfx950.
//
// What it computes ("cortex-engine write-up", model section and kernels section, fused spike
// tokenizer): each spike event (neuron id, time bin, value) of a row becomes a token whose
// embedding is the sum of three table rows, x = (n_emb[neuron] + t_emb[bin]) + v_emb[value] in
// fp32; its key and value are x . W_k^T and x . W_v^T, split into the pool's heads and stored at
// the token's slot through the row's block table ("NeuroGrid releases", v0.7.0 "Paged KV Cache").
// The embeddings never go to HBM: they are built in LDS and fed to the matrix cores.
//
// Mapping: one workgroup (8 waves) per kTB consecutive 16-token blocks of one row.
//   1. The blocks' event ids go to LDS; then each thread takes float4 pieces of the tokens'
//      embeddings (consecutive lanes, consecutive float4s of a row, so a quarter-wave reads 256
//      contiguous bytes of each table), adds the three, rounds to bf16 (the matrix-core input)
//      and parks the result in LDS: X [16 kTB][Dm].
//   2. The output columns (H * dh of K, then as many of V) are cut into 16-wide tiles; wave w
//      owns tiles w, w + 8, ..., taken kT at a time. A tile is computed as W_tile . X^T with
//      v_mfma_f32_16x16x32_bf16 (fp32 accumulation): operand A is the weight slice (output
//      column lane % 16, 8 consecutive inputs), operand B the tokens (token lane % 16, the same 8
//      inputs, from LDS). The loop runs over 32-input steps: per step a wave reads its kTB token
//      fragments from LDS once and applies them to its kT tiles' weight fragments, so each LDS
//      read feeds kT products and each weight fragment kTB. The weights come pre-packed in
//      fragment order (pack_projection_kernel): a fragment is 64 lanes x 16 contiguous bytes,
//      one coalesced 1 KB read, where the [out][in] layout would make every quarter-wave touch 16
//      rows. Two steps of weight fragments are in flight, the first two requested before the
//      embeddings are built.
//   3. Lane l of an accumulator holds output columns 4 (l / 16) .. + 3 of token l % 16: rounded
//      to bf16 they are 8 contiguous bytes of the token's slot [block][head][slot][dim].
#include <map>
#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTB = 4;           // 16-token blocks per workgroup
constexpr int kTok = 16 * kTB;   // tokens per workgroup
constexpr int kWaves = 8;
constexpr int kMaxDm = 512;      // LDS holds X [kTok][kMaxDm + 8] bf16
constexpr int kT = 4;            // tiles a wave carries through one pass over the inputs
constexpr int kEmbedUnroll = 2;  // float4 pieces in flight per thread while embedding
// With PRE (launches the device holds at once), a wave whose steps number at most kPre requests
// all their weight fragments at the start, before the embedding, instead of two steps ahead: its
// products then never wait on a load (the model width 256 gives 8 steps). That takes 254 VGPRs,
// one workgroup per CU, so larger launches keep the two-step pipeline at two workgroups per CU.
constexpr int kPre = 8;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return (unsigned)__builtin_bit_cast(unsigned short, static_cast<__bf16>(lo)) |
         ((unsigned)__builtin_bit_cast(unsigned short, static_cast<__bf16>(hi)) << 16);
}

struct Step {
  u32x4_t w[kT];  // the kT tiles' weight fragments for one 32-input step
};

template <bool PRE>
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
  // the pool block of each 16-token sub-block, read now so that its latency hides behind the
  // embedding (entry (t0 >> 4) + b, clamped into the row's bt_stride entries: t0 < n <=
  // bt_stride * 16, and a sub-block past the row's end is never stored)
  int bids[kTB];
#pragma unroll
  for (int b = 0; b < kTB; ++b) {
    const int e = (t0 >> 4) + b < a.bt_stride ? (t0 >> 4) + b : a.bt_stride - 1;
    bids[b] = a.block_tables[(size_t)row * a.bt_stride + e];
  }

  // the wave's steps: tile group g (tiles wave + kWaves (kT g + i), i < kT) x input step kc
  const int N = a.H * a.dh;  // columns of K (and of V)
  const int tiles = 2 * N / 16;
  const int my_tiles = tiles > wave ? (tiles - wave + kWaves - 1) / kWaves : 0;
  const int groups = (my_tiles + kT - 1) / kT;
  const int nk = Dm / 32;  // 32-input steps per tile
  const int steps = groups * nk;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // step j's fragments: packed fragment (tile within K or V, kc), this lane's 16 bytes. Every load
  // is unconditional (a conditional one would make each later wait drain all loads): tiles past
  // the wave's last and steps past the end read the first fragment of W_k instead, unused.
  auto load_step = [&](Step& st, int j) {
    const int g = j / nk;
    const int kc = j - g * nk;
    const u32x4_t* w0 = reinterpret_cast<const u32x4_t*>(a.w_k) + lane;
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const int tile = wave + kWaves * (kT * g + i);
      const bool live = j < steps && tile < tiles;
      const bool is_v = tile * 16 >= N;
      const int tk = tile - (is_v ? N / 16 : 0);
      const u32x4_t* w = reinterpret_cast<const u32x4_t*>(is_v ? a.w_v : a.w_k) +
                         ((size_t)tk * nk + kc) * 64 + lane;
      st.w[i] = *(live ? w : w0);  // one load, through the chosen address
    }
  };
  Step sa, sb;
  Step pre[PRE ? kPre : 1];
  bool pre_all = false;  // uniform
  if constexpr (PRE) {
    pre_all = steps <= kPre;
    if (pre_all) {
#pragma unroll
      for (int j = 0; j < kPre; ++j) load_step(pre[j], j);
    }
  }
  if (!pre_all && steps > 0) {
    load_step(sa, 0);
    load_step(sb, 1);
  }

  // 1. event ids of the tokens (tokens past nt: row 0 of each table, never stored)
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
    // piece p: token p / (Dm / 4), float4 p % (Dm / 4) of its row; kEmbedUnroll pieces per thread
    // are loaded before any is used (their addresses are always inside the tables)
    const int f4 = Dm / 4;
    const int pieces = kTok * f4;
    for (int base = tid; base < pieces; base += kEmbedUnroll * 64 * kWaves) {
      float4 xn[kEmbedUnroll], xt[kEmbedUnroll], xv[kEmbedUnroll];
#pragma unroll
      for (int u = 0; u < kEmbedUnroll; ++u) {
        const int p = base + u * 64 * kWaves;
        const int t = p / f4 < kTok ? p / f4 : kTok - 1;
        const int f = p - (p / f4) * f4;
        xn[u] = reinterpret_cast<const float4*>(a.n_emb + (size_t)s_ids[t][0] * Dm)[f];
        xt[u] = reinterpret_cast<const float4*>(a.t_emb + (size_t)s_ids[t][1] * Dm)[f];
        xv[u] = reinterpret_cast<const float4*>(a.v_emb + (size_t)s_ids[t][2] * Dm)[f];
      }
#pragma unroll
      for (int u = 0; u < kEmbedUnroll; ++u) {
        const int p = base + u * 64 * kWaves;
        if (p < pieces) {
          const int t = p / f4;
          const int f = p - t * f4;
          uint2 r = make_uint2(0u, 0u);
          if (t < nt) {
            // (n + t) + v, each sum one fp32 operation
            r.x = pack_bf16x2((xn[u].x + xt[u].x) + xv[u].x, (xn[u].y + xt[u].y) + xv[u].y);
            r.y = pack_bf16x2((xn[u].z + xt[u].z) + xv[u].z, (xn[u].w + xt[u].w) + xv[u].w);
          }
          *reinterpret_cast<uint2*>(&s_x[t][4 * f]) = r;
        }
      }
    }
  }
  __syncthreads();

  // 2. the projection
  // Branch-free except for the stores (branches around loads or products would leave the
  // compiler unsure which loads are outstanding, and it would then wait for all of them): tiles
  // past the wave's last and the padding step multiply the dummy fragment and are never stored,
  // and the accumulators are cleared right after each group's stores.
  f32x4_t acc[kT][kTB];
#pragma unroll
  for (int i = 0; i < kT; ++i)
#pragma unroll
    for (int b = 0; b < kTB; ++b) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute_step = [&](const Step& st, int j) {
    const int g = j / nk;
    const int kc = j - g * nk;
    u32x4_t xb[kTB];
#pragma unroll
    for (int b = 0; b < kTB; ++b)
      xb[b] = *reinterpret_cast<const u32x4_t*>(&s_x[16 * b + col][32 * kc + 8 * grp]);
#pragma unroll
    for (int i = 0; i < kT; ++i)
#pragma unroll
      for (int b = 0; b < kTB; ++b)
        acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, st.w[i]), __builtin_bit_cast(bf16x8_t, xb[b]), acc[i][b],
            0, 0, 0);
    if (kc == nk - 1) {
      // 3. store: lane holds columns c .. c + 3 (one head) of token 16 b + col
#pragma unroll
      for (int i = 0; i < kT; ++i) {
        const int tile = wave + kWaves * (kT * g + i);
        if (tile < tiles) {
          const bool is_v = tile * 16 >= N;
          const int c = tile * 16 - (is_v ? N : 0) + 4 * grp;
          const int head = c / a.dh;
          const int dim = c % a.dh;
          __bf16* pool = reinterpret_cast<__bf16*>(is_v ? a.v : a.k);
#pragma unroll
          for (int b = 0; b < kTB; ++b) {
            const int t = 16 * b + col;
            if (t < nt) {
              // tokens of sub-block b live in the row's block (t0 >> 4) + b
              const int bid = clampi(bids[b], 0, a.num_blocks - 1);
              *reinterpret_cast<uint2*>(
                  pool + (((size_t)bid * a.H + head) * kBlock + (t & 15)) * a.dh + dim) =
                  make_uint2(pack_bf16x2(acc[i][b][0], acc[i][b][1]),
                             pack_bf16x2(acc[i][b][2], acc[i][b][3]));
            }
          }
        }
#pragma unroll
        for (int b = 0; b < kTB; ++b) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // two steps in flight: while one computes, the next is already on its way (the step count is
  // padded to even; the padding step is a dummy)
  if constexpr (PRE) {
    if (pre_all) {
#pragma unroll
      for (int j = 0; j < kPre; ++j)
        if (j < steps) compute_step(pre[j], j);
      return;
    }
  }
  const int steps2 = steps + (steps & 1);
  for (int j = 0; j < steps2; j += 2) {
    compute_step(sa, j);
    load_step(sa, j + 2);
    compute_step(sb, j + 1);
    load_step(sb, j + 3);
  }
}

// packed[((tile * nk + kc) * 64 + lane) * 8 + j] = w[16 tile + lane % 16][32 kc + 8 (lane / 16) + j]:
// the A-operand fragment of v_mfma_f32_16x16x32_bf16 for output tile `tile`, inputs 32 kc .. + 31.
// One thread per lane-fragment (16 bytes).
__global__ __launch_bounds__(256) void pack_projection_kernel(const u32x4_t* __restrict__ w,
                                                             u32x4_t* __restrict__ packed,
                                                             int out_features, int in_features) {
  const int nk = in_features / 32;
  const size_t total = (size_t)(out_features / 16) * nk * 64;
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= total) return;
  const int lane = (int)(g & 63);
  const size_t frag = g >> 6;
  const int tile = (int)(frag / nk);
  const int kc = (int)(frag % nk);
  const int r = 16 * tile + (lane & 15);
  const int k0 = 32 * kc + 8 * (lane >> 4);
  packed[g] = w[((size_t)r * in_features + k0) / 8];
}

}  // namespace

int tokenize_max_model_dim() { return kMaxDm; }

// Workgroups of the prefetching instance the current device holds at once (0 if unknown), cached
// per device.
static int resident_prefetching() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(tokenize_kv_kernel<true>), 64 * kWaves, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cache[dev] = per_cu * cus;
  return per_cu * cus;
}

hipError_t launch_tokenize(const TokenizeArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.max_events <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.max_events + kTok - 1) / kTok), (unsigned)a.batch);
  const long long wgs = (long long)grid.x * grid.y;
  const int resident = resident_prefetching();
  if (resident > 0 && wgs <= resident)
    hipLaunchKernelGGL((tokenize_kv_kernel<true>), grid, dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((tokenize_kv_kernel<false>), grid, dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pack_projection(const void* w, void* packed, int out_features, int in_features,
                                  hipStream_t stream) {
  const size_t total = (size_t)(out_features / 16) * (in_features / 32) * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_projection_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, reinterpret_cast<const u32x4_t*>(w), reinterpret_cast<u32x4_t*>(packed),
                     out_features, in_features);
  return hipGetLastError();
}

}  // namespace pa
