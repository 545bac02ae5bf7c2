// cvt_exhaust.hip -- device check of the kernels' FP8 encode step against
// the oracle, over every fp32 bit pattern.
//
// The MXFP8 kernels turn an fp32 value into an FP8 code by a clamp to
// +-FP8_MAX (sat_clamp), then the gfx950 packed conversion (cvt4), four
// values per dword.  This program runs exactly those two helpers from
// fp8q_device.h on the GPU for all 2^32 fp32 patterns, in both formats, and
// compares each code with the oracle's integer-exact satRNE
// (oracle_fp8_encode: round to nearest, ties to even, saturating, signed zero
// kept) on the host.  NaN patterns are not compared: no kernel converts a
// NaN (a block holding a non-finite value writes 0x7F codes without
// converting), and the oracle's NaN code is a reading of its own.
//
// The same program checks the bf16 outputs' rounding: bf16_pack2 (the
// kernels' fp32 -> bf16 store conversion) on the device against the oracle's
// f32_to_bf16 (round to nearest even, overflow to inf), again for all 2^32
// fp32 patterns.  Here NaN inputs can reach the conversion (a NaN code or
// scale makes a NaN sum); the oracle reads every NaN as 0x7FC0, and NaN
// patterns are counted apart ("bf16 nan: ... differ").
//
// Two more passes check the encode of the block-scale kernels, which
// convert their quotients without the clamp: cvt4 alone against the oracle
// for every fp32 in [-quotient_bound, quotient_bound].  A last pass checks
// the MXFP8 receiver's scaled decode (mx_dec2) for every E4M3 code and every
// E8M0 scale against the oracle's MXFP8 dequantize; NaN results are compared
// as NaN.
//
// Output: one line per pass, then "values: N mismatches: M" over the
// non-NaN patterns of all passes.  Exit status 0 only when all of those
// agree.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "fp8q_device.h"

extern "C" uint8_t oracle_fp8_encode(double y, int fmt);
extern "C" uint16_t oracle_f32_to_bf16(float f);
extern "C" int oracle_mx8_dequantize(const uint8_t *q, const uint8_t *e8m0, size_t rows, size_t K,
                                     void *y, int out_bf16);

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

// The same without the clamp: the block-scale kernels (block quantize,
// tensorwise, requantize) convert their quotients with cvt4 alone, since a
// quotient never exceeds quotient_bound in magnitude.  Compared on
// [-quotient_bound, quotient_bound] only.
template <int FMT>
__global__ __launch_bounds__(256) void encode_patterns_unclamped(uint32_t first, uint32_t *out,
                                                                 uint32_t words) {
  for (uint32_t w = blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += gridDim.x * blockDim.x) {
    const uint32_t b = first + 4u * w;
    out[w] = fp8q::cvt4<FMT>(__uint_as_float(b), __uint_as_float(b + 1u),
                             __uint_as_float(b + 2u), __uint_as_float(b + 3u));
  }
}

// The MXFP8 receiver's scaled decode (mx_dec2): for pair t = 256 c + b, the
// E4M3 code b in all four bytes of a dword and the E8M0 scale code c, both
// halves of the packed conversion (4 values per pair).
__global__ __launch_bounds__(256) void mx_dec_pairs(uint32_t *out) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;         // 256 x 256 launch: t < 65536
  const uint32_t b = t & 255u, c = t >> 8;
  const uint32_t w = b * 0x01010101u;
  const fp8q::f32x2 lo = fp8q::mx_dec2<false>(w, c), hi = fp8q::mx_dec2<true>(w, c);
  out[4 * t + 0] = __float_as_uint(lo[0]);
  out[4 * t + 1] = __float_as_uint(lo[1]);
  out[4 * t + 2] = __float_as_uint(hi[0]);
  out[4 * t + 3] = __float_as_uint(hi[1]);
}

// Word w of the chunk holds the bf16 of patterns first + 2w (low half) and
// first + 2w + 1 (high half).  first + 2w + 1 <= 2^32 - 1 for every chunk.
__global__ __launch_bounds__(256) void bf16_patterns(uint32_t first, uint32_t *out,
                                                     uint32_t words) {
  for (uint32_t w = blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += gridDim.x * blockDim.x) {
    const uint32_t b = first + 2u * w;
    out[w] = fp8q::bf16_pack2(__uint_as_float(b), __uint_as_float(b + 1u));
  }
}

bool is_nan_pattern(uint32_t b) { return (b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu); }

struct Tally {
  uint64_t compared = 0, mismatches = 0;   // non-NaN patterns
  uint64_t nan_compared = 0, nan_differ = 0;
  uint32_t first_bad = 0, first_nan_differ = 0;
  uint32_t got = 0, want = 0, nan_got = 0;
};

// Host comparison of one chunk of n patterns from `first`, split over
// threads.  fmt 0 / 1: FP8 codes (one byte each, NaN patterns skipped);
// fmt 2: bf16 (two bytes each, NaN patterns counted apart).
Tally compare_chunk(const uint8_t *out, uint32_t first, uint32_t n, int fmt, unsigned threads) {
  std::vector<Tally> part(threads);
  std::vector<std::thread> pool;
  for (unsigned t = 0; t < threads; ++t) {
    pool.emplace_back([&, t] {
      const uint32_t lo = (uint32_t)((uint64_t)n * t / threads);
      const uint32_t hi = (uint32_t)((uint64_t)n * (t + 1) / threads);
      Tally &r = part[t];
      for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t b = first + i;
        float v;
        memcpy(&v, &b, 4);
        uint32_t got, want;
        if (fmt < 2) {
          if (is_nan_pattern(b)) continue;
          got = out[i];
          want = oracle_fp8_encode((double)v, fmt);
        } else {
          uint16_t h;
          memcpy(&h, out + 2 * (size_t)i, 2);
          got = h;
          want = oracle_f32_to_bf16(v);
          if (is_nan_pattern(b)) {
            ++r.nan_compared;
            if (got != want && r.nan_differ++ == 0) {
              r.first_nan_differ = b;
              r.nan_got = got;
            }
            continue;
          }
        }
        ++r.compared;
        if (got != want) {
          if (r.mismatches == 0) {
            r.first_bad = b;
            r.got = got;
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
    if (r.nan_differ && !sum.nan_differ) {
      sum.first_nan_differ = r.first_nan_differ;
      sum.nan_got = r.nan_got;
    }
    sum.compared += r.compared;
    sum.mismatches += r.mismatches;
    sum.nan_compared += r.nan_compared;
    sum.nan_differ += r.nan_differ;
  }
  return sum;
}

}  // namespace

int main() {
  unsigned threads = std::thread::hardware_concurrency();
  threads = std::max(1u, std::min(threads, 16u));
  uint32_t *d_out = nullptr;
  CHECK(hipMalloc(&d_out, (size_t)kChunkWords * 4));
  std::vector<uint8_t> out((size_t)kChunkWords * 4);
  uint64_t total_compared = 0, total_bad = 0;
  const char *names[3] = {"e4m3", "e5m2", "bf16"};
  for (int pass = 0; pass < 3; ++pass) {
    // patterns per chunk: 4 per word for the FP8 passes, 2 for bf16
    const uint64_t per_chunk = (pass < 2 ? 4ull : 2ull) * kChunkWords;
    Tally all;
    for (uint64_t first = 0; first < (1ull << 32); first += per_chunk) {
      if (pass == 0)
        hipLaunchKernelGGL(encode_patterns<0>, dim3(4096), dim3(256), 0, 0, (uint32_t)first,
                           d_out, kChunkWords);
      else if (pass == 1)
        hipLaunchKernelGGL(encode_patterns<1>, dim3(4096), dim3(256), 0, 0, (uint32_t)first,
                           d_out, kChunkWords);
      else
        hipLaunchKernelGGL(bf16_patterns, dim3(4096), dim3(256), 0, 0, (uint32_t)first, d_out,
                           kChunkWords);
      CHECK(hipGetLastError());
      CHECK(hipMemcpy(out.data(), d_out, out.size(), hipMemcpyDeviceToHost));
      const Tally t = compare_chunk(out.data(), (uint32_t)first, (uint32_t)per_chunk, pass,
                                    threads);
      if (t.mismatches && !all.mismatches)
        printf("  first mismatch: pattern 0x%08X got 0x%02X want 0x%02X\n", t.first_bad, t.got,
               t.want);
      if (t.nan_differ && !all.nan_differ)
        printf("  first NaN that differs: pattern 0x%08X got 0x%04X\n", t.first_nan_differ,
               t.nan_got);
      all.compared += t.compared;
      all.mismatches += t.mismatches;
      all.nan_compared += t.nan_compared;
      all.nan_differ += t.nan_differ;
    }
    printf("%s: compared %llu fp32 patterns (all but NaN), mismatches %llu\n", names[pass],
           (unsigned long long)all.compared, (unsigned long long)all.mismatches);
    if (pass == 2)
      printf("bf16 nan: %llu NaN patterns, %llu differ from 0x7FC0\n",
             (unsigned long long)all.nan_compared, (unsigned long long)all.nan_differ);
    fflush(stdout);
    total_compared += all.compared;
    total_bad += all.mismatches;
  }
  // The unclamped encode on [-B, B], B = quotient_bound (both signs; the
  // ranges end below 0xD8000000, so first + 4w + 3 never wraps).
  const char *unames[2] = {"e4m3 unclamped", "e5m2 unclamped"};
  for (int fmt = 0; fmt < 2; ++fmt) {
    const float bnd = fmt == 0 ? fp8q::quotient_bound<0>() : fp8q::quotient_bound<1>();
    uint32_t bb;
    memcpy(&bb, &bnd, 4);
    const uint64_t per_chunk = 4ull * kChunkWords;
    Tally all;
    for (int sign = 0; sign < 2; ++sign) {
      const uint64_t lo = sign ? 0x80000000ull : 0ull, hi = lo + bb;   // inclusive
      for (uint64_t first = lo; first <= hi; first += per_chunk) {
        if (fmt == 0)
          hipLaunchKernelGGL(encode_patterns_unclamped<0>, dim3(4096), dim3(256), 0, 0,
                             (uint32_t)first, d_out, kChunkWords);
        else
          hipLaunchKernelGGL(encode_patterns_unclamped<1>, dim3(4096), dim3(256), 0, 0,
                             (uint32_t)first, d_out, kChunkWords);
        CHECK(hipGetLastError());
        CHECK(hipMemcpy(out.data(), d_out, out.size(), hipMemcpyDeviceToHost));
        const uint64_t cnt = std::min<uint64_t>(per_chunk, hi - first + 1);
        const Tally t = compare_chunk(out.data(), (uint32_t)first, (uint32_t)cnt, fmt, threads);
        if (t.mismatches && !all.mismatches)
          printf("  first mismatch: pattern 0x%08X got 0x%02X want 0x%02X\n", t.first_bad, t.got,
                 t.want);
        all.compared += t.compared;
        all.mismatches += t.mismatches;
      }
    }
    printf("%s: compared %llu fp32 patterns in [-%08X, %08X], mismatches %llu\n", unames[fmt],
           (unsigned long long)all.compared, bb, bb, (unsigned long long)all.mismatches);
    fflush(stdout);
    total_compared += all.compared;
    total_bad += all.mismatches;
  }
  // The MXFP8 scaled decode against the oracle's MXFP8 dequantize of a
  // [256, 256] matrix whose row c holds every code b and has all its E8M0
  // scales equal to c.
  {
    hipLaunchKernelGGL(mx_dec_pairs, dim3(256), dim3(256), 0, 0, d_out);
    CHECK(hipGetLastError());
    std::vector<uint32_t> got(4 * 65536);
    CHECK(hipMemcpy(got.data(), d_out, got.size() * 4, hipMemcpyDeviceToHost));
    std::vector<uint8_t> q(65536), e(256 * 8);
    for (uint32_t i = 0; i < 65536; ++i) q[i] = (uint8_t)(i & 255u);
    for (uint32_t i = 0; i < 256 * 8; ++i) e[i] = (uint8_t)(i / 8);
    std::vector<float> want(65536);
    if (oracle_mx8_dequantize(q.data(), e.data(), 256, 256, want.data(), 0) != 0) return 2;
    uint64_t cmp = 0, bad = 0, nan = 0;
    for (uint32_t t = 0; t < 65536; ++t) {
      uint32_t wb;
      memcpy(&wb, &want[t], 4);
      for (int j = 0; j < 4; ++j) {
        const uint32_t g = got[4 * t + j];
        ++cmp;
        if (is_nan_pattern(wb) || is_nan_pattern(g)) {
          ++nan;
          if (is_nan_pattern(wb) != is_nan_pattern(g)) ++bad;
        } else if (g != wb) {
          if (!bad)
            printf("  first mismatch: code 0x%02X scale %u got 0x%08X want 0x%08X\n", t & 255u,
                   t >> 8, g, wb);
          ++bad;
        }
      }
    }
    printf("mx scaled decode: compared %llu values (every code x every E8M0 scale, 4 positions), "
           "NaN %llu, mismatches %llu\n", (unsigned long long)cmp, (unsigned long long)nan,
           (unsigned long long)bad);
    fflush(stdout);
    total_compared += cmp;
    total_bad += bad;
  }
  CHECK(hipFree(d_out));
  printf("values: %llu mismatches: %llu\n", (unsigned long long)total_compared,
         (unsigned long long)total_bad);
  return total_bad == 0 ? 0 : 1;
}
