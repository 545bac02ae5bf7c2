/* The largest quotient the block-scale kernels ever convert, over every
 * finite amax.
 *
 * The block quantize, the tensorwise quantize and the requantize encode
 * RN(x / s) with s = max(RN(amax / M), 2^-126), M = 448 (e4m3) or 57344
 * (e5m2), where amax is the block's (or tensor's) largest |x|.  They hand
 * that quotient to the hardware FP8 conversion with no clamp.  Rounding is
 * monotone and odd, so |RN(x / s)| <= RN(amax / s) for every x of the block;
 * this program computes RN(amax / s) with IEEE divides for every finite
 * non-negative fp32 amax (2^31 - 2^23 values, which include every bf16
 * amax) and checks that it never exceeds B = M (1 + 2^-23), the next fp32
 * above M.  It also reports whether B is reached.  It shares no code with
 * the kernels or the oracle.  Prints "over: N" (patterns above B) and exits
 * with status 1 when N > 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  const float M[2] = {448.0f, 57344.0f};
  const char *name[2] = {"e4m3", "e5m2"};
  unsigned long long over_all = 0;
  for (int k = 0; k < 2; ++k) {
    const uint32_t bound = bits_of(M[k]) + 1u;      /* M (1 + 2^-23) */
    unsigned long long over = 0, at_bound = 0, at_max = 0;
#pragma omp parallel for reduction(+ : over, at_bound, at_max) schedule(static, 1 << 16)
    for (int64_t i = 0; i < 0x7F800000LL; ++i) {
      const float amax = from_bits((uint32_t)i);
      const float s = fmaxf(amax / M[k], 0x1p-126f);
      const uint32_t qb = bits_of(amax / s);
      if (qb > bound) ++over;
      if (qb == bound) ++at_bound;
      if (qb == bits_of(M[k])) ++at_max;
    }
    printf("%s: amax values %lld, bound %08x, over: %llu, quotient = bound for %llu, = M for %llu\n",
           name[k], 0x7F800000LL, bound, over, at_bound, at_max);
    over_all += over;
  }
  printf("over: %llu\n", over_all);
  return over_all ? 1 : 0;
}
