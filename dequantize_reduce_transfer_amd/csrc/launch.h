// launch.h -- internal launchers behind the C ABI (not exported).
//
// Each launcher assumes the arguments were validated by the C-ABI layer
// (non-null, aligned, non-overlapping, 0 < n <= FP8Q_MAX_ELEMS) and only
// sizes the grid and enqueues the kernel on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int kMaxPeers = 16;

// Block-128 quantize of n bf16 values (fmt 0 = E4M3, 1 = E5M2).
hipError_t launch_quantize(int fmt, const void *x, uint64_t n, void *q, float *scales,
                           hipStream_t stream, int num_cus);

// Fused dequantize-then-reduce of k shards (k == 1 is a dequantize).
hipError_t launch_dequant_reduce(int fmt, int k, bool out_bf16, const void *const *q,
                                 const float *const *scales, uint64_t n, void *y,
                                 hipStream_t stream, int num_cus);

// Ordered sum of k fp32 arrays (the naive path's reduction).
hipError_t launch_sum_f32(int k, bool out_bf16, const float *const *parts, uint64_t n, void *y,
                          hipStream_t stream, int num_cus);

// MXFP8 quantize of n bf16 values laid out as [rows, K] with K % 32 == 0.
hipError_t launch_mx8_quantize(const void *w, uint64_t n, void *q, void *e8m0,
                               hipStream_t stream, int num_cus);

}  // namespace fp8q
