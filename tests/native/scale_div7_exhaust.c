/* The divide-free block scale, restated on the host, against the IEEE divide.
 *
 * The kernels compute s = max(RN(amax / M), 2^-126), M = 448 (e4m3) or 57344
 * (e5m2), without a divide: M = 7 * 2^m, so with c = RN(1/7)
 *   q0 = RN(amax * c),  r = fma(-q0, 7, amax),  t = fma(r, c, q0),
 *   s  = max(RN(t * 2^-m), 2^-126).
 * This program checks t == RN(amax / 7) and s == max(RN(amax / M), 2^-126)
 * for every finite non-negative fp32 amax (2^31 - 2^23 values), in hardware
 * fp32 with fma and no contraction.  It shares no code with the kernels or
 * the oracle.  Prints "mismatches: N"; exit status 1 when N > 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  const float c = 1.0f / 7.0f;
  const float M[2] = {448.0f, 57344.0f};
  const float P[2] = {0x1p-6f, 0x1p-13f};
  if (bits_of(c) != 0x3E124925u) { printf("RN(1/7) is %08x\n", bits_of(c)); return 2; }
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 16)
  for (int64_t i = 0; i < 0x7F800000LL; ++i) {
    const float a = from_bits((uint32_t)i);
    const float q0 = a * c;
    const float r = fmaf(-q0, 7.0f, a);
    const float t = fmaf(r, c, q0);
    if (bits_of(t) != bits_of(a / 7.0f)) ++bad;
    for (int k = 0; k < 2; ++k)
      if (bits_of(fmaxf(t * P[k], 0x1p-126f)) != bits_of(fmaxf(a / M[k], 0x1p-126f))) ++bad;
  }
  printf("inputs: %lld\nmismatches: %llu\n", 0x7F800000LL, bad);
  return bad ? 1 : 0;
}
