// cvt_exhaust.hip -- device check of the kernels' FP8 encode step against
// the oracle, over every fp32 bit pattern.
//
// Every kernel turns an fp32 value into an FP8 code the same way: clamp to
// +-FP8_MAX (sat_clamp), then the gfx950 packed conversion (cvt4), four
// values per dword.  This program runs exactly those two helpers from
// fp8q_device.h on the GPU for all 2^32 fp32 patterns, in both formats, and
// compares each code with the oracle's integer-exact satRNE
// (oracle_fp8_encode: round to nearest, ties to even, saturating, signed zero
// kept) on the host.  NaN patterns are not compared: no kernel converts a
// NaN (a block holding a non-finite value writes 0x7F codes without
// converting), and the oracle's NaN code is a reading of its own.
//
// Output: one line per format, then "values: N mismatches: M".  Exit status
// 0 only when every compared pattern agrees.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "fp8q_device.h"

extern "C" uint8_t oracle_fp8_encode(double y, int fmt);

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                  \
      return 2;                                                                       \
    }                                                                                 \
  } while (0)

namespace {

constexpr uint32_t kChunkWords = 1u << 26;   // 2^28 patterns per chunk, 4 per word

// Word w of the chunk holds the codes of patterns first + 4w .. first + 4w + 3
// (byte j <- pattern first + 4w + j), so both halves of each packed
// conversion are exercised.  first + 4w + 3 <= 2^32 - 1 for every chunk.
template <int FMT>
__global__ __launch_bounds__(256) void encode_patterns(uint32_t first, uint32_t *out,
                                                       uint32_t words) {
  for (uint32_t w = blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += gridDim.x * blockDim.x) {
    const uint32_t b = first + 4u * w;
    out[w] = fp8q::cvt4<FMT>(fp8q::sat_clamp<FMT>(__uint_as_float(b)),
                             fp8q::sat_clamp<FMT>(__uint_as_float(b + 1u)),
                             fp8q::sat_clamp<FMT>(__uint_as_float(b + 2u)),
                             fp8q::sat_clamp<FMT>(__uint_as_float(b + 3u)));
  }
}

bool is_nan_pattern(uint32_t b) { return (b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu); }

struct Tally {
  uint64_t compared = 0, mismatches = 0;
  uint32_t first_bad = 0;
  uint8_t got = 0, want = 0;
};

// Host comparison of one chunk, split over threads.
Tally compare_chunk(const uint8_t *codes, uint32_t first, int fmt, unsigned threads) {
  const uint32_t n = 4u * kChunkWords;
  std::vector<Tally> part(threads);
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < threads; ++t) {
    pool.emplace_back([&, t] {
      const uint32_t lo = (uint32_t)((uint64_t)n * t / threads);
      const uint32_t hi = (uint32_t)((uint64_t)n * (t + 1) / threads);
      Tally &r = part[t];
      for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t b = first + i;
        if (is_nan_pattern(b)) continue;
        float v;
        memcpy(&v, &b, 4);
        const uint8_t want = oracle_fp8_encode((double)v, fmt);
        ++r.compared;
        if (codes[i] != want) {
          if (r.mismatches == 0) {
            r.first_bad = b;
            r.got = codes[i];
            r.want = want;
          }
          ++r.mismatches;
        }
      }
    });
  }
  for (auto &th : pool) th.join();
  Tally sum;
  for (const Tally &r : part) {
    if (r.mismatches && !sum.mismatches) {
      sum.first_bad = r.first_bad;
      sum.got = r.got;
      sum.want = r.want;
    }
    sum.compared += r.compared;
    sum.mismatches += r.mismatches;
  }
  return sum;
}

}  // namespace

int main() {
  unsigned threads = std::thread::hardware_concurrency();
  threads = std::max(1u, std::min(threads, 16u));
  uint32_t *d_out = nullptr;
  CHECK(hipMalloc(&d_out, (size_t)kChunkWords * 4));
  std::vector<uint8_t> codes((size_t)kChunkWords * 4);
  uint64_t total_compared = 0, total_bad = 0;
  for (int fmt = 0; fmt < 2; ++fmt) {
    uint64_t compared = 0, bad = 0;
    for (uint64_t first = 0; first < (1ull << 32); first += 4ull * kChunkWords) {
      if (fmt == 0)
        hipLaunchKernelGGL(encode_patterns<0>, dim3(4096), dim3(256), 0, 0, (uint32_t)first,
                           d_out, kChunkWords);
      else
        hipLaunchKernelGGL(encode_patterns<1>, dim3(4096), dim3(256), 0, 0, (uint32_t)first,
                           d_out, kChunkWords);
      CHECK(hipGetLastError());
      CHECK(hipMemcpy(codes.data(), d_out, codes.size(), hipMemcpyDeviceToHost));
      const Tally t = compare_chunk(codes.data(), (uint32_t)first, fmt, threads);
      if (t.mismatches && !bad)
        printf("  first mismatch: pattern 0x%08X got 0x%02X want 0x%02X\n", t.first_bad, t.got,
               t.want);
      compared += t.compared;
      bad += t.mismatches;
    }
    printf("%s: compared %llu fp32 patterns (all but NaN), mismatches %llu\n",
           fmt == 0 ? "e4m3" : "e5m2", (unsigned long long)compared, (unsigned long long)bad);
    fflush(stdout);
    total_compared += compared;
    total_bad += bad;
  }
  CHECK(hipFree(d_out));
  printf("values: %llu mismatches: %llu\n", (unsigned long long)total_compared,
         (unsigned long long)total_bad);
  return total_bad == 0 ? 0 : 1;
}
