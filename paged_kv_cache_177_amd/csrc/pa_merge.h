// Internal interface of the log-sum-exp merge of partial attention results (pa_merge.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct LseMergeArgs {
  const float* out_parts;  // [num_parts][n][D]
  const float* lse_parts;  // [num_parts][n], natural log
  int num_parts;
  long long n;             // (row, query head) pairs
  int D;
  float* out;              // [n][D]
  float* lse;              // [n] or NULL
};

hipError_t launch_lse_merge(const LseMergeArgs& a, hipStream_t stream);

}  // namespace pa
