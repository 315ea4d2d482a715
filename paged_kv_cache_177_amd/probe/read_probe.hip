// HBM read-ceiling probe for the benchmark (a measuring instrument, not part of the attention
// library): every workgroup streams its share of a large device buffer with 16-byte
// non-temporal loads, four in flight per lane, and folds them into one word, so the launch's
// duration gives the practical read bandwidth to compare the decode kernels with.
#include <hip/hip_runtime.h>

#include "pa_probe.h"

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4_t* __restrict__ p,
                                                              size_t n16, unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  unsigned acc = 0;
  // main part: kUnroll unconditional loads per iteration
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the fold keeps the loads; one word per thread goes out (sink holds grid * kThreads words)
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int pa_probe_read(const void* buf, size_t bytes, unsigned* sink, int grid,
                             hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || grid < 1 || bytes % 16 != 0 ||
      (uintptr_t)buf % 16 != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}
