// api.hip -- the C ABI declared in include/fp8q.h: host-side validation,
// grid sizing and dispatch to the gfx950 kernels.
//
// Every check runs before anything is enqueued, in this order: enums and
// counts, size limit, null pointers, alignment, overlap.  A failed check
// returns its status with no launch, so no output byte is ever written by a
// rejected call (the boundary rejects bad requests before any work, as the
// prequantized-refit handshake does in "perf: Reduce MXFP8 refit
// weight-transfer overheads", section "Safety").  The library never
// allocates device memory: every buffer is the caller's.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fp8q.h"
#include "launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t num_blocks(size_t n, size_t block) { return (n + block - 1) / block; }

bool valid_fmt(fp8q_format f) { return f == FP8Q_E4M3 || f == FP8Q_E5M2; }
bool valid_out(fp8q_out_dtype d) { return d == FP8Q_OUT_F32 || d == FP8Q_OUT_BF16; }
size_t out_elem_bytes(fp8q_out_dtype d) { return d == FP8Q_OUT_F32 ? 4 : 2; }

fp8q_status from_hip(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_HIP; }

}  // namespace

extern "C" {

fp8q_status fp8q_quantize(const void *x_bf16, size_t n, fp8q_format fmt, void *q_out,
                          float *scales_out, void *stream) {
  if (!valid_fmt(fmt)) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (n > FP8Q_MAX_ELEMS) return FP8Q_ERR_ARG;
  if (!x_bf16 || !q_out || !scales_out) return FP8Q_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scales_out, 4)) return FP8Q_ERR_ALIGN;
  const size_t sb = 4 * num_blocks(n, FP8Q_BLOCK);
  if (overlaps(x_bf16, 2 * n, q_out, n) || overlaps(x_bf16, 2 * n, scales_out, sb) ||
      overlaps(q_out, n, scales_out, sb))
    return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_quantize((int)fmt, x_bf16, n, q_out, scales_out,
                                        static_cast<hipStream_t>(stream)));
}

fp8q_status fp8q_dequant_reduce(const void *const *q_peers, const float *const *scales_peers, int k,
                                size_t n, fp8q_format fmt, void *y_out, fp8q_out_dtype out_dtype,
                                void *stream) {
  if (!valid_fmt(fmt) || !valid_out(out_dtype)) return FP8Q_ERR_ARG;
  if (k < 1 || k > FP8Q_MAX_PEERS) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (n > FP8Q_MAX_ELEMS) return FP8Q_ERR_ARG;
  if (!q_peers || !scales_peers || !y_out) return FP8Q_ERR_NULL;
  for (int p = 0; p < k; ++p)
    if (!q_peers[p] || !scales_peers[p]) return FP8Q_ERR_NULL;
  if (!aligned(y_out, 16)) return FP8Q_ERR_ALIGN;
  for (int p = 0; p < k; ++p)
    if (!aligned(q_peers[p], 16) || !aligned(scales_peers[p], 4)) return FP8Q_ERR_ALIGN;
  const size_t yb = out_elem_bytes(out_dtype) * n;
  const size_t sb = 4 * num_blocks(n, FP8Q_BLOCK);
  for (int p = 0; p < k; ++p)
    if (overlaps(y_out, yb, q_peers[p], n) || overlaps(y_out, yb, scales_peers[p], sb))
      return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_dequant_reduce((int)fmt, k, out_dtype == FP8Q_OUT_BF16, q_peers,
                                              scales_peers, n, y_out,
                                              static_cast<hipStream_t>(stream)));
}

fp8q_status fp8q_dequantize(const void *q, const float *scales, size_t n, fp8q_format fmt,
                            void *y_out, fp8q_out_dtype out_dtype, void *stream) {
  if (!valid_fmt(fmt) || !valid_out(out_dtype)) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (!q || !scales) return FP8Q_ERR_NULL;
  const void *qp[1] = {q};
  const float *sp[1] = {scales};
  return fp8q_dequant_reduce(qp, sp, 1, n, fmt, y_out, out_dtype, stream);
}

fp8q_status mx8_quantize(const void *w_bf16, size_t rows, size_t K, void *q_out, void *e8m0_out,
                         void *stream) {
  if (K % FP8Q_MX_BLOCK != 0) return FP8Q_ERR_ARG;
  if (rows == 0 || K == 0) return FP8Q_OK;
  if (rows > FP8Q_MAX_ELEMS || K > FP8Q_MAX_ELEMS || rows > FP8Q_MAX_ELEMS / K)
    return FP8Q_ERR_ARG;
  const size_t n = rows * K;
  if (!w_bf16 || !q_out || !e8m0_out) return FP8Q_ERR_NULL;
  if (!aligned(w_bf16, 16) || !aligned(q_out, 16)) return FP8Q_ERR_ALIGN;
  const size_t eb = n / FP8Q_MX_BLOCK;
  if (overlaps(w_bf16, 2 * n, q_out, n) || overlaps(w_bf16, 2 * n, e8m0_out, eb) ||
      overlaps(q_out, n, e8m0_out, eb))
    return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_mx8_quantize(w_bf16, n, q_out, e8m0_out,
                                            static_cast<hipStream_t>(stream)));
}

fp8q_status fp8q_sum_f32(const float *const *parts, int k, size_t n, void *y_out,
                         fp8q_out_dtype out_dtype, void *stream) {
  if (!valid_out(out_dtype)) return FP8Q_ERR_ARG;
  if (k < 1 || k > FP8Q_MAX_PEERS) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (n > FP8Q_MAX_ELEMS) return FP8Q_ERR_ARG;
  if (!parts || !y_out) return FP8Q_ERR_NULL;
  for (int p = 0; p < k; ++p)
    if (!parts[p]) return FP8Q_ERR_NULL;
  if (!aligned(y_out, 16)) return FP8Q_ERR_ALIGN;
  for (int p = 0; p < k; ++p)
    if (!aligned(parts[p], 16)) return FP8Q_ERR_ALIGN;
  const size_t yb = out_elem_bytes(out_dtype) * n;
  for (int p = 0; p < k; ++p)
    if (overlaps(y_out, yb, parts[p], 4 * n)) return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_sum_f32(k, out_dtype == FP8Q_OUT_BF16, parts, n, y_out,
                                       static_cast<hipStream_t>(stream)));
}

fp8q_status fp8q_dequant_reduce_requantize(const void *const *q_peers,
                                           const float *const *scales_peers, int k, size_t n,
                                           fp8q_format fmt_in, fp8q_format fmt_out, void *q_out,
                                           float *scales_out, void *stream) {
  if (!valid_fmt(fmt_in) || !valid_fmt(fmt_out)) return FP8Q_ERR_ARG;
  if (k < 1 || k > FP8Q_MAX_PEERS) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (n > FP8Q_MAX_ELEMS) return FP8Q_ERR_ARG;
  if (!q_peers || !scales_peers || !q_out || !scales_out) return FP8Q_ERR_NULL;
  for (int p = 0; p < k; ++p)
    if (!q_peers[p] || !scales_peers[p]) return FP8Q_ERR_NULL;
  if (!aligned(q_out, 16) || !aligned(scales_out, 4)) return FP8Q_ERR_ALIGN;
  for (int p = 0; p < k; ++p)
    if (!aligned(q_peers[p], 16) || !aligned(scales_peers[p], 4)) return FP8Q_ERR_ALIGN;
  const size_t sb = 4 * num_blocks(n, FP8Q_BLOCK);
  if (overlaps(q_out, n, scales_out, sb)) return FP8Q_ERR_OVERLAP;
  for (int p = 0; p < k; ++p)
    if (overlaps(q_out, n, q_peers[p], n) || overlaps(q_out, n, scales_peers[p], sb) ||
        overlaps(scales_out, sb, q_peers[p], n) || overlaps(scales_out, sb, scales_peers[p], sb))
      return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_reduce_requantize((int)fmt_in, (int)fmt_out, k, q_peers,
                                                 scales_peers, n, q_out, scales_out,
                                                 static_cast<hipStream_t>(stream)));
}

fp8q_status mx8_dequant_reduce(const void *const *q_peers, const void *const *e8m0_peers, int k,
                               size_t rows, size_t K, void *y_out, fp8q_out_dtype out_dtype,
                               void *stream) {
  if (!valid_out(out_dtype)) return FP8Q_ERR_ARG;
  if (k < 1 || k > FP8Q_MAX_PEERS) return FP8Q_ERR_ARG;
  if (K % FP8Q_MX_BLOCK != 0) return FP8Q_ERR_ARG;
  if (rows == 0 || K == 0) return FP8Q_OK;
  if (rows > FP8Q_MAX_ELEMS || K > FP8Q_MAX_ELEMS || rows > FP8Q_MAX_ELEMS / K)
    return FP8Q_ERR_ARG;
  const size_t n = rows * K;
  if (!q_peers || !e8m0_peers || !y_out) return FP8Q_ERR_NULL;
  for (int p = 0; p < k; ++p)
    if (!q_peers[p] || !e8m0_peers[p]) return FP8Q_ERR_NULL;
  if (!aligned(y_out, 16)) return FP8Q_ERR_ALIGN;
  for (int p = 0; p < k; ++p)
    if (!aligned(q_peers[p], 16)) return FP8Q_ERR_ALIGN;
  const size_t yb = out_elem_bytes(out_dtype) * n;
  const size_t eb = n / FP8Q_MX_BLOCK;
  for (int p = 0; p < k; ++p)
    if (overlaps(y_out, yb, q_peers[p], n) || overlaps(y_out, yb, e8m0_peers[p], eb))
      return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_mx8_dequant_reduce(k, out_dtype == FP8Q_OUT_BF16, q_peers,
                                                  e8m0_peers, n, y_out,
                                                  static_cast<hipStream_t>(stream)));
}

fp8q_status mx8_dequantize(const void *q, const void *e8m0, size_t rows, size_t K, void *y_out,
                           fp8q_out_dtype out_dtype, void *stream) {
  if (!valid_out(out_dtype)) return FP8Q_ERR_ARG;
  if (K % FP8Q_MX_BLOCK != 0) return FP8Q_ERR_ARG;
  if (rows == 0 || K == 0) return FP8Q_OK;
  if (!q || !e8m0) return FP8Q_ERR_NULL;
  const void *qp[1] = {q};
  const void *ep[1] = {e8m0};
  return mx8_dequant_reduce(qp, ep, 1, rows, K, y_out, out_dtype, stream);
}

fp8q_status fp8q_quantize_tensorwise(const void *x_bf16, size_t n, fp8q_format fmt, void *q_out,
                                     float *scale_out, void *stream) {
  if (!valid_fmt(fmt)) return FP8Q_ERR_ARG;
  if (n == 0) return FP8Q_OK;
  if (n > FP8Q_MAX_ELEMS) return FP8Q_ERR_ARG;
  if (!x_bf16 || !q_out || !scale_out) return FP8Q_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4)) return FP8Q_ERR_ALIGN;
  if (overlaps(x_bf16, 2 * n, q_out, n) || overlaps(x_bf16, 2 * n, scale_out, 4) ||
      overlaps(q_out, n, scale_out, 4))
    return FP8Q_ERR_OVERLAP;
  return from_hip(fp8q::launch_quantize_tensorwise((int)fmt, x_bf16, n, q_out, scale_out,
                                                   static_cast<hipStream_t>(stream)));
}

const char *fp8q_status_str(fp8q_status s) {
  switch (s) {
    case FP8Q_OK: return "FP8Q_OK: success";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: a required pointer is NULL";
    case FP8Q_ERR_ARG: return "FP8Q_ERR_ARG: invalid format, dtype, peer count, K or size";
    case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN: a pointer breaks the alignment rule";
    case FP8Q_ERR_OVERLAP: return "FP8Q_ERR_OVERLAP: an output range overlaps another range";
    case FP8Q_ERR_HIP: return "FP8Q_ERR_HIP: the HIP runtime reported an error";
  }
  return "FP8Q: unknown status";
}

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

}  // extern "C"
