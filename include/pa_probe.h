/*
 * pa_probe.h -- the benchmark's HBM read-ceiling probe (libpa_probe.so). A measuring instrument
 * that bench.py uses to report the practical read bandwidth next to the decode kernels' figures;
 * it is not part of the attention library's ABI.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Read all `bytes` of the device buffer `buf` (16-byte aligned, bytes a multiple of 16) with a
 * grid of `grid` workgroups of 256 threads, each thread folding what it reads into one word that
 * it writes to sink[workgroup * 256 + thread] (device, grid * 256 words, caller-owned). Returns 0
 * (hipSuccess) or the HIP error code (hipErrorInvalidValue for bad arguments, nothing launched).
 * Asynchronous on stream. */
int pa_probe_read(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
