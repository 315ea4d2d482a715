// Merge of partial attention results computed over disjoint key sets, for gfx950: the step after
// an all-gather when one long row's keys are split across GPUs.
//
// Each part p holds, for every (row, query head) n, the part's normalised output o_p[n][0..D) and
// its log-sum-exp l_p[n] (natural log; -inf for a part with no keys). The merged result is
//   M = max_p l_p,  w_p = exp(l_p - M),  out = sum_p w_p o_p / sum_p w_p,  lse = M + log sum_p w_p
// -- the same algebra as the library's own split-K merge of a long row's chunks (the pages never
// split a row, so this step is the library's design, not theirs), with a part of weight 0 dropping
// out and out = 0, lse = -inf when every part is empty. Parts are summed in
// index order, so the result does not depend on the launch geometry.
//
// One wave per (row, head) n: lane i owns dims i and i + 64. The parts' lse values are read 64 at a
// time (one per lane) and their maximum and weights formed across the wave; the part outputs are
// read in batches of 8 (the first batch together with the lse values, so a merge of a few parts
// waits for one round of loads), and each weight is broadcast from its lane as they are summed.
#include "pa_merge.h"

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

__global__ __launch_bounds__(256) void lse_merge_kernel(const LseMergeArgs a) {
  constexpr int kBatch = 8;  // part outputs in flight at once
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.n) return;  // whole waves
  const int P = a.num_parts;
  const int D = a.D;
  // this lane's dims of parts p0 .. p0 + kBatch - 1 (indices clamped to the last part; the extra
  // slots are never summed)
  float v0[kBatch], v1[kBatch];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = p0 + i < P ? p0 + i : P - 1;
      const float* o = a.out_parts + ((size_t)p * a.n + n) * D;
      v0[i] = lane < D ? o[lane] : 0.f;
      v1[i] = D > 64 ? o[64 + lane] : 0.f;
    }
  };
  // the first batch of outputs goes in flight with the parts' lse values
  load_batch(0);
  float mx = kNegInf;
  for (int p = lane; p < P; p += 64) mx = fmaxf(mx, a.lse_parts[(size_t)p * a.n + n]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
  if (mx != kNegInf) {
    for (int p0 = 0; p0 < P; p0 += 64) {
      const int p = p0 + lane;
      const float l = p < P ? a.lse_parts[(size_t)p * a.n + n] : kNegInf;
      const float w = l == kNegInf ? 0.f : expf(l - mx);
      const int cnt = P - p0 < 64 ? P - p0 : 64;
      for (int k = 0; k < cnt; k += kBatch) {
        if (p0 + k > 0) load_batch(p0 + k);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          if (k + i < cnt) {  // uniform
            const float wi = __shfl(w, k + i);
            wsum += wi;
            acc0 = fmaf(wi, v0[i], acc0);
            acc1 = fmaf(wi, v1[i], acc1);
          }
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* out = a.out + (size_t)n * D;
  if (lane < D) out[lane] = acc0 * inv;
  if (D > 64) out[64 + lane] = acc1 * inv;
  if (a.lse != nullptr && lane == 0) a.lse[n] = wsum > 0.f ? mx + logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_lse_merge(const LseMergeArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const long long blocks = (a.n + 3) / 4;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
