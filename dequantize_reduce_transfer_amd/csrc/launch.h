// launch.h -- internal launchers behind the C ABI (not exported).
//
// Each launcher assumes the arguments were validated by the C-ABI layer
// (non-null, aligned, non-overlapping, 0 < n <= FP8Q_MAX_ELEMS) and only
// sizes the grid and enqueues the kernel on `stream`.
//
// Tuning constants (tile depths, streaming hints) are compile-time macros
// with the defaults chosen by measurement on MI355X at the full workload
// sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int kMaxPeers = 16;

// Grid size: one workgroup of waves_per_wg waves per waves_per_wg units of
// wave work (the argument counts those units: tiles, or groups of T tiles),
// so that the tiles in flight at any moment form one window of the buffer
// (measured faster on MI355X than a persistent grid, whose waves drift apart
// across the whole buffer; the workgroup -> position map inside the window
// is XCD-aware, see block_position in fp8q_device.h).  The cap keeps
// grid * 256 work-items inside the dispatch packet's 32-bit range; beyond it
// the kernels' grid-stride loops take the rest.
#ifndef FP8Q_MAX_WORKGROUPS
#define FP8Q_MAX_WORKGROUPS (1ull << 22)
#endif
constexpr uint64_t kMaxWorkgroups = FP8Q_MAX_WORKGROUPS;

inline uint32_t grid_for_tiles(uint64_t tiles, uint32_t waves_per_wg = 4) {
  uint64_t wgs = (tiles + waves_per_wg - 1) / waves_per_wg;
  if (wgs > kMaxWorkgroups) wgs = kMaxWorkgroups;
  if (wgs < 1) wgs = 1;
  return (uint32_t)wgs;
}

// Block-128 quantize of n bf16 values (fmt 0 = E4M3, 1 = E5M2).
hipError_t launch_quantize(int fmt, const void *x, uint64_t n, void *q, float *scales,
                           hipStream_t stream);

// Tensorwise quantize: one fp32 scale for the whole tensor, written to
// *scale (which also serves as the amax slot while the kernels run).
hipError_t launch_quantize_tensorwise(int fmt, const void *x, uint64_t n, void *q, float *scale,
                                      hipStream_t stream);

// Fused dequantize-then-reduce of k shards (k == 1 is a dequantize).
hipError_t launch_dequant_reduce(int fmt, int k, bool out_bf16, const void *const *q,
                                 const float *const *scales, uint64_t n, void *y,
                                 hipStream_t stream);

// Dequant-reduce of k shards, then block-128 requantize of the fp32 sums.
hipError_t launch_reduce_requantize(int fmt_in, int fmt_out, int k, const void *const *q,
                                   const float *const *scales, uint64_t n, void *q_out,
                                   float *scales_out, hipStream_t stream);

// MXFP8 dequant-reduce of k shards of n = rows * K elements (k == 1: dequantize).
hipError_t launch_mx8_dequant_reduce(int k, bool out_bf16, const void *const *q,
                                     const void *const *e8m0, uint64_t n, void *y,
                                     hipStream_t stream);

// Ordered sum of k fp32 arrays (the naive path's reduction).
hipError_t launch_sum_f32(int k, bool out_bf16, const float *const *parts, uint64_t n, void *y,
                          hipStream_t stream);

// MXFP8 quantize of n bf16 values laid out as [rows, K] with K % 32 == 0.
hipError_t launch_mx8_quantize(const void *w, uint64_t n, void *q, void *e8m0,
                               hipStream_t stream);

}  // namespace fp8q
