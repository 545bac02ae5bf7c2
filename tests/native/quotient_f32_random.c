/*
 * The kernels' divide-free quotient of an fp32 dividend against the IEEE
 * fp32 divide, on random and adversarial pairs (fp32 arithmetic with
 * explicit fmaf; built with -ffp-contract=off):
 *   y = 1/b (IEEE);  q0 = a*y;  e0 = fma(q0, b, -a);  q1 = fma(-e0, y, q0);
 *   claim: q1 == a/b.
 * Pairs: (1) random significands and exponents with |a/b| in [2^-40, 2^10];
 * (2) adversarial: b random, a = fl(m * b) +- up to 3 ulps for m a random
 * fp32 midpoint (an odd multiple of half an ulp), so a/b sits next to a
 * rounding boundary; (3) signed zeros.  Usage: prog <count> <seed>.
 * Prints the mismatch count; exit status 1 if any.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st;
static uint64_t nxt(void) { st ^= st >> 12; st ^= st << 25; st ^= st >> 27; return st * 0x2545F4914F6CDD1Dull; }
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float seq(float a, float b) {
  volatile float y = 1.0f / b;
  float q0 = a * y;
  volatile float e0 = fmaf(q0, b, -a);
  return fmaf(-e0, y, q0);
}

static long check(float a, float b) {
  float want = a / b, got = seq(a, b);
  if (u_of(want) != u_of(got)) {
    if (getenv("VERBOSE")) fprintf(stderr, "a=%a b=%a want=%a got=%a\n", a, b, want, got);
    return 1;
  }
  return 0;
}

int main(int argc, char **argv) {
  long count = argc > 1 ? atol(argv[1]) : 100000000L;
  st = argc > 2 ? strtoull(argv[2], 0, 10) * 0x9E3779B97F4A7C15ull + 1 : 88172645463325252ull;
  long bad = 0;
  for (long i = 0; i < count; ++i) {
    uint64_t r = nxt();
    uint32_t sb = (uint32_t)(r & 0x7FFFFF), sa = (uint32_t)((r >> 23) & 0x7FFFFF);
    int eb = (int)((r >> 46) % 120) - 60;             /* b in [2^-60, 2^60) */
    int gap = (int)((r >> 53) % 51) - 40;             /* |a/b| ~ 2^gap */
    float b = ldexpf(f_of(0x3F800000u | sb), eb);
    float a = ldexpf(f_of(0x3F800000u | sa), eb + gap);
    if (r >> 63) a = -a;
    bad += check(a, b);
    /* adversarial: a/b next to a rounding boundary of the quotient */
    uint64_t r2 = nxt();
    uint32_t mq = (uint32_t)(r2 & 0x7FFFFF);
    double m = ldexp(1.0 + ldexp((double)mq, -23) + ldexp(1.0, -24), (int)((r2 >> 23) % 21) - 10);
    float a2 = (float)(m * (double)b);                 /* RN to fp32 */
    int d = (int)((r2 >> 40) % 7) - 3;
    uint32_t ua = u_of(a2) + (uint32_t)d;
    a2 = f_of(ua);
    if (isfinite(a2) && a2 != 0.0f) bad += check((r2 >> 63) ? -a2 : a2, b);
  }
  bad += check(0.0f, 3.0f) + check(-0.0f, 3.0f) + check(0.0f, 0x1p-126f) + check(-0.0f, 0x1p-100f);
  printf("pairs=%ld mismatches=%ld\n", 2 * count + 4, bad);
  return bad ? 1 : 0;
}
