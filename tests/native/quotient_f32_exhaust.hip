// Device proof by exhaustion of the kernels' quotient (markstein_quotient in
// fp8q_device.h, one Markstein step): for every pair of fp32 significands, x
// and s in [1, 2) (2^23 x 2^23 pairs), markstein_quotient(x, s, recip_rn(s))
// equals hipcc's IEEE fp32 divide x / s.  Every operation in the sequence is exact under scaling by a
// power of two while its results stay normal, so these pairs stand for all
// normal x and s with normal intermediates; the sequence is odd in x, so
// negative x behaves the same.
//
// Usage: quotient_f32_exhaust [s_count]  (the first s_count significands of s,
// default all 2^23).  Runs in launches of 2^17 s values, printing progress;
// prints "mismatches: N" and exits 1 when N > 0, 2 when a HIP call fails.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fp8q_device.h"

namespace {

constexpr uint32_t kSig = 1u << 23;            // significands per binade
constexpr uint32_t kXPerThread = 1u << 13;     // x values one thread walks
constexpr uint32_t kSPerLaunch = 1u << 17;     // s values per launch
constexpr uint32_t kFirstBad = 16;

// blockIdx.x: which run of kXPerThread x significands; blockIdx.y * 256 +
// threadIdx.x: which s significand (offset by s0).
__global__ __launch_bounds__(256) void check(uint32_t s0, uint32_t s_count,
                                             unsigned long long *cnt, uint32_t *bad) {
  const uint32_t is = s0 + blockIdx.y * 256u + threadIdx.x;
  if (is >= s_count) return;
  const float s = __uint_as_float(0x3F800000u | is);
  const float rp = fp8q::recip_rn(s);
  const uint32_t x0 = blockIdx.x * kXPerThread;
  for (uint32_t j = 0; j < kXPerThread; ++j) {
    const uint32_t ix = x0 + j;
    const float x = __uint_as_float(0x3F800000u | ix);
    const float q = fp8q::markstein_quotient(x, s, rp);
    if (__float_as_uint(q) != __float_as_uint(x / s)) {
      const unsigned long long k = atomicAdd(cnt, 1ull);
      if (k < kFirstBad) {
        bad[2 * k] = ix;
        bad[2 * k + 1] = is;
      }
    }
  }
}

}  // namespace

#define CHECK(call)                                                     \
  do {                                                                  \
    hipError_t e_ = (call);                                             \
    if (e_ != hipSuccess) {                                             \
      printf("%s failed: %s\n", #call, hipGetErrorString(e_));          \
      return 2;                                                         \
    }                                                                   \
  } while (0)

int main(int argc, char **argv) {
  uint32_t s_count = kSig;
  if (argc > 1) {
    const long v = strtol(argv[1], nullptr, 10);
    if (v < 1 || v > (long)kSig) {
      printf("s_count must be in [1, %u]\n", kSig);
      return 2;
    }
    s_count = (uint32_t)v;
  }
  unsigned long long *cnt = nullptr;
  uint32_t *bad = nullptr;
  CHECK(hipMalloc(&cnt, sizeof(unsigned long long)));
  CHECK(hipMalloc(&bad, 2 * kFirstBad * sizeof(uint32_t)));
  CHECK(hipMemset(cnt, 0, sizeof(unsigned long long)));
  const uint32_t launches = (s_count + kSPerLaunch - 1) / kSPerLaunch;
  for (uint32_t l = 0; l < launches; ++l) {
    const uint32_t s0 = l * kSPerLaunch;
    const uint32_t n = s_count - s0 < kSPerLaunch ? s_count - s0 : kSPerLaunch;
    hipLaunchKernelGGL(check, dim3(kSig / kXPerThread, (n + 255) / 256), dim3(256), 0, 0, s0,
                       s_count, cnt, bad);
    CHECK(hipGetLastError());
    if ((l + 1) % 8 == 0 || l + 1 == launches) {
      CHECK(hipDeviceSynchronize());
      printf("s significands done: %u of %u\n", s0 + n, s_count);
      fflush(stdout);
    }
  }
  unsigned long long h = 0;
  uint32_t hb[2 * kFirstBad];
  CHECK(hipMemcpy(&h, cnt, sizeof h, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(hb, bad, sizeof hb, hipMemcpyDeviceToHost));
  for (unsigned long long i = 0; i < h && i < kFirstBad; ++i)
    printf("differs: x = 1 + %u * 2^-23, s = 1 + %u * 2^-23\n", hb[2 * i], hb[2 * i + 1]);
  printf("pairs: %llu\nmismatches: %llu\n", (unsigned long long)s_count * kSig, h);
  CHECK(hipFree(cnt));
  CHECK(hipFree(bad));
  return h ? 1 : 0;
}
