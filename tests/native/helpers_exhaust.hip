// Device check of the kernels' divide-free helpers (fp8q_device.h) against
// the IEEE fp32 divide, on the GPU that runs them:
//   scale_from_amax<E4M3/E5M2>(a) == max(a / M, 2^-126)  for every finite a >= 0;
//   recip_rn(x) == 1 / x  for every normal x with a normal reciprocal
//                          (x in [2^-126, 2^126)).
// The IEEE divides are hipcc's correctly rounded fp32 division.  Prints
// "mismatches: N" (and the first few inputs that differ); exit status 1 when
// N > 0, 2 when a HIP call fails.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "fp8q_device.h"

namespace {

constexpr uint32_t kFirstBad = 16;

__device__ void record(unsigned long long *cnt, uint32_t *bad, uint32_t what, uint32_t bits) {
  const unsigned long long k = atomicAdd(cnt, 1ull);
  if (k < kFirstBad) {
    bad[2 * k] = what;
    bad[2 * k + 1] = bits;
  }
}

__global__ void check_scale(uint64_t n, unsigned long long *cnt, uint32_t *bad) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t bits = (uint32_t)i;                     // 0 .. 0x7F7FFFFF
  const float a = __uint_as_float(bits);
  const float s4 = fp8q::scale_from_amax<0>(a), r4 = fmaxf(a / 448.0f, 0x1p-126f);
  const float s5 = fp8q::scale_from_amax<1>(a), r5 = fmaxf(a / 57344.0f, 0x1p-126f);
  if (__float_as_uint(s4) != __float_as_uint(r4)) record(cnt, bad, 0, bits);
  if (__float_as_uint(s5) != __float_as_uint(r5)) record(cnt, bad, 1, bits);
}

__global__ void check_recip(uint64_t n, unsigned long long *cnt, uint32_t *bad) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t bits = 0x00800000u + (uint32_t)i;      // 2^-126 .. below 2^126
  const float x = __uint_as_float(bits);
  if (__float_as_uint(fp8q::recip_rn(x)) != __float_as_uint(1.0f / x)) record(cnt, bad, 2, bits);
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

int main() {
  const uint64_t n_scale = 0x7F800000ull;                // finite non-negative fp32
  const uint64_t n_recip = 0x7E800000ull - 0x00800000ull;
  unsigned long long *cnt = nullptr;
  uint32_t *bad = nullptr;
  CHECK(hipMalloc(&cnt, sizeof(unsigned long long)));
  CHECK(hipMalloc(&bad, 2 * kFirstBad * sizeof(uint32_t)));
  CHECK(hipMemset(cnt, 0, sizeof(unsigned long long)));
  // grids of 256-thread workgroups; every thread past n returns at once
  hipLaunchKernelGGL(check_scale, dim3((uint32_t)((n_scale + 255) / 256)), dim3(256), 0, 0,
                     n_scale, cnt, bad);
  CHECK(hipGetLastError());
  hipLaunchKernelGGL(check_recip, dim3((uint32_t)((n_recip + 255) / 256)), dim3(256), 0, 0,
                     n_recip, cnt, bad);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  unsigned long long h = 0;
  uint32_t hb[2 * kFirstBad];
  CHECK(hipMemcpy(&h, cnt, sizeof h, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(hb, bad, sizeof hb, hipMemcpyDeviceToHost));
  const char *names[3] = {"scale e4m3", "scale e5m2", "recip"};
  for (unsigned long long i = 0; i < h && i < kFirstBad; ++i)
    printf("differs: %s at %08x\n", names[hb[2 * i] % 3], hb[2 * i + 1]);
  printf("inputs: scale %llu, recip %llu\nmismatches: %llu\n", (unsigned long long)n_scale,
         (unsigned long long)n_recip, h);
  CHECK(hipFree(cnt));
  CHECK(hipFree(bad));
  return h ? 1 : 0;
}
