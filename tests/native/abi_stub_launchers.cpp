// abi_stub_launchers.cpp -- host-only stand-ins for the kernel launchers, so
// that the C-ABI layer (csrc/api.hip, compiled host-only with g++) can run
// under AddressSanitizer and UndefinedBehaviorSanitizer on a machine without
// a GPU.
//
// Each stub enqueues nothing.  It checks the invariants the real launchers
// assume of a validated call (launch.h): non-null, suitably aligned and
// pairwise disjoint buffers, 0 < n <= FP8Q_MAX_ELEMS, 1 <= k <= 16, known
// formats.  Then it records the call.  A broken invariant returns
// hipErrorInvalidValue, which the ABI reports as FP8Q_ERR_HIP, so a
// validation gap shows up as a wrong status in the tests.  The peer arrays
// are read element by element, so a short host array is a sanitizer report.
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp8q.h"

namespace {

struct Record {
  long calls;
  char last[32];
  uint64_t n;
  int k;
};
Record g_rec = {0, {0}, 0, 0};

bool al(const void *p, uintptr_t a) { return p && reinterpret_cast<uintptr_t>(p) % a == 0; }

bool disjoint(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x + na <= y || y + nb <= x;
}

uint64_t blocks(uint64_t n, uint64_t b) { return (n + b - 1) / b; }

bool size_ok(uint64_t n) { return n > 0 && n <= FP8Q_MAX_ELEMS; }

hipError_t record(const char *name, uint64_t n, int k) {
  ++g_rec.calls;
  strncpy(g_rec.last, name, sizeof(g_rec.last) - 1);
  g_rec.n = n;
  g_rec.k = k;
  return hipSuccess;
}

// Every peer's inputs are present and aligned, and none overlaps the outputs
// [o1, o1 + n1) and [o2, o2 + n2).
bool peers_ok(int k, const void *const *q, const void *const *s, uintptr_t s_align, uint64_t qn,
              uint64_t sn, const void *o1, uint64_t n1, const void *o2, uint64_t n2) {
  if (k < 1 || k > FP8Q_MAX_PEERS || !q || !s) return false;
  for (int p = 0; p < k; ++p) {
    if (!al(q[p], 16) || !al(s[p], s_align)) return false;
    if (!disjoint(q[p], qn, o1, n1) || !disjoint(s[p], sn, o1, n1)) return false;
    if (o2 && (!disjoint(q[p], qn, o2, n2) || !disjoint(s[p], sn, o2, n2))) return false;
  }
  return true;
}

}  // namespace

namespace fp8q {

hipError_t launch_quantize(int fmt, const void *x, uint64_t n, void *q, float *scales,
                           hipStream_t) {
  const uint64_t sb = 4 * blocks(n, FP8Q_BLOCK);
  if ((fmt != 0 && fmt != 1) || !size_ok(n) || !al(x, 16) || !al(q, 16) || !al(scales, 4) ||
      !disjoint(x, 2 * n, q, n) || !disjoint(x, 2 * n, scales, sb) || !disjoint(q, n, scales, sb))
    return hipErrorInvalidValue;
  return record("quantize", n, 1);
}

hipError_t launch_quantize_tensorwise(int fmt, const void *x, uint64_t n, void *q, float *scale,
                                      hipStream_t) {
  if ((fmt != 0 && fmt != 1) || !size_ok(n) || !al(x, 16) || !al(q, 16) || !al(scale, 4) ||
      !disjoint(x, 2 * n, q, n) || !disjoint(x, 2 * n, scale, 4) || !disjoint(q, n, scale, 4))
    return hipErrorInvalidValue;
  return record("quantize_tensorwise", n, 1);
}

hipError_t launch_dequant_reduce(int fmt, int k, bool out_bf16, const void *const *q,
                                 const float *const *scales, uint64_t n, void *y, hipStream_t) {
  const uint64_t yb = (out_bf16 ? 2 : 4) * n;
  if ((fmt != 0 && fmt != 1) || !size_ok(n) || !al(y, 16) ||
      !peers_ok(k, q, reinterpret_cast<const void *const *>(scales), 4, n,
                4 * blocks(n, FP8Q_BLOCK), y, yb, nullptr, 0))
    return hipErrorInvalidValue;
  return record(k == 1 ? "dequantize" : "dequant_reduce", n, k);
}

hipError_t launch_reduce_requantize(int fmt_in, int fmt_out, int k, const void *const *q,
                                    const float *const *scales, uint64_t n, void *q_out,
                                    float *scales_out, hipStream_t) {
  const uint64_t sb = 4 * blocks(n, FP8Q_BLOCK);
  if ((fmt_in != 0 && fmt_in != 1) || (fmt_out != 0 && fmt_out != 1) || !size_ok(n) ||
      !al(q_out, 16) || !al(scales_out, 4) || !disjoint(q_out, n, scales_out, sb) ||
      !peers_ok(k, q, reinterpret_cast<const void *const *>(scales), 4, n, sb, q_out, n,
                scales_out, sb))
    return hipErrorInvalidValue;
  return record("reduce_requantize", n, k);
}

hipError_t launch_mx8_dequant_reduce(int k, bool out_bf16, const void *const *q,
                                     const void *const *e8m0, uint64_t n, void *y, hipStream_t) {
  const uint64_t yb = (out_bf16 ? 2 : 4) * n;
  if (!size_ok(n) || n % FP8Q_MX_BLOCK || !al(y, 16) ||
      !peers_ok(k, q, e8m0, 1, n, n / FP8Q_MX_BLOCK, y, yb, nullptr, 0))
    return hipErrorInvalidValue;
  return record(k == 1 ? "mx8_dequantize" : "mx8_dequant_reduce", n, k);
}

hipError_t launch_sum_f32(int k, bool out_bf16, const float *const *parts, uint64_t n, void *y,
                          hipStream_t) {
  const uint64_t yb = (out_bf16 ? 2 : 4) * n;
  if (k < 1 || k > FP8Q_MAX_PEERS || !parts || !size_ok(n) || !al(y, 16)) return hipErrorInvalidValue;
  for (int p = 0; p < k; ++p)
    if (!al(parts[p], 16) || !disjoint(parts[p], 4 * n, y, yb)) return hipErrorInvalidValue;
  return record("sum_f32", n, k);
}

hipError_t launch_mx8_quantize(const void *w, uint64_t n, void *q, void *e8m0, hipStream_t) {
  const uint64_t eb = n / FP8Q_MX_BLOCK;
  if (!size_ok(n) || n % FP8Q_MX_BLOCK || !al(w, 16) || !al(q, 16) || !e8m0 ||
      !disjoint(w, 2 * n, q, n) || !disjoint(w, 2 * n, e8m0, eb) || !disjoint(q, n, e8m0, eb))
    return hipErrorInvalidValue;
  return record("mx8_quantize", n, 1);
}

}  // namespace fp8q

// Read back by the tests (ctypes) when the library under test is the
// host-check build.
extern "C" __attribute__((visibility("default"))) long fp8q_stub_calls(void) { return g_rec.calls; }
extern "C" __attribute__((visibility("default"))) const char *fp8q_stub_last(void) {
  return g_rec.last;
}
extern "C" __attribute__((visibility("default"))) unsigned long long fp8q_stub_last_n(void) {
  return g_rec.n;
}
extern "C" __attribute__((visibility("default"))) int fp8q_stub_last_k(void) { return g_rec.k; }
