/*
 * Exhaustive check, in emulated p-bit binary floating point (p = 8 .. 13),
 * of the divide-free quotient the kernels use:
 *   y  = RN(1/b)
 *   q0 = RN(a * y)
 *   r0 = RN(a - b * q0)      (fused multiply-add)
 *   q1 = RN(q0 + r0 * y)     (fused multiply-add)
 * claim: q1 == RN(a / b) for every pair of p-bit significands a, b in
 * [1, 2) (every step is invariant under power-of-two scaling, so this
 * covers every pair of normal numbers whose intermediates stay normal).
 * It also reports a second correction step,
 *   r1 = RN(a - b * q1),  q2 = RN(q1 + r1 * y),
 * which Markstein's theorem proves correctly rounded on paper.
 * p-bit arithmetic is emulated in double: every product and sum of p-bit
 * values here needs at most 3p < 53 bits, so the double result is exact and
 * a single rounding to p bits reproduces one p-bit operation.  The exact
 * quotient is never within 2^-53 of a p-bit midpoint unless equal to it, so
 * RN_p(double(a / b)) is RN_p(a / b).
 * Prints the number of mismatches per p; exit status 1 if either sequence
 * has any.
 */
#include <math.h>
#include <stdio.h>

static int P;
#ifndef PMIN
#define PMIN 8
#endif
#ifndef PMAX
#define PMAX 13
#endif

static double rn(double x) {      /* round to nearest even, P significant bits */
  if (x == 0.0) return x;
  int e;
  double m = frexp(x, &e);        /* x = m * 2^e, 0.5 <= |m| < 1 */
  return ldexp(nearbyint(ldexp(m, P)), e - P);
}

int main(void) {
  int bad_total = 0;
  for (P = PMIN; P <= PMAX; ++P) {
    long n = 1L << (P - 1), bad = 0, one_step_bad = 0;
    for (long i = 0; i < n; ++i) {
      const double a = 1.0 + ldexp((double)i, 1 - P);
      for (long j = 0; j < n; ++j) {
        const double b = 1.0 + ldexp((double)j, 1 - P);
        const double y = rn(1.0 / b);
        const double q0 = rn(a * y);
        const double r0 = rn(a - b * q0);
        const double q1 = rn(q0 + r0 * y);
        const double r1 = rn(a - b * q1);
        const double q2 = rn(q1 + r1 * y);
        const double want = rn(a / b);
        if (q2 != want) ++bad;
        if (q1 != want) ++one_step_bad;
      }
    }
    printf("p=%2d pairs=%ld two-step mismatches=%ld one-step mismatches=%ld\n", P, n * n, bad,
           one_step_bad);
    bad_total += (bad != 0) + (one_step_bad != 0);
  }
  return bad_total ? 1 : 0;
}
