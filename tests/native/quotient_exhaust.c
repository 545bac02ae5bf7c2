/*
 * Exhaustive host check of the block-128 quantize kernel's quotient.
 *
 * The kernel never divides per element.  Per block it forms
 *   s  = max(fl32(amax / M), 2^-126),  f = (amax < 2^-60) ? 2^64 : 1,
 *   sp = s * f,  rp = RN(1 / sp)
 * and per element, with x' = x * f:
 *   q0 = RN(x' * rp);  e = RN(q0 * sp - x') (fma);  q1 = RN(q0 - e * rp) (fma)
 * The definition needs RN(x / s).  This program checks, on the CPU with IEEE
 * fp32 and hardware fma:
 *  (1) q1 == x / s bit for bit for every pair (bf16 significand of x, fp32
 *      significand of s) -- 128 * 2^23 pairs.  Both sides are invariant under
 *      x -> x 2^a, s -> s 2^b while every intermediate stays normal, so this
 *      covers the whole normal range;
 *  (2) over every pair of bf16 exponents (x <= amax), every x significand
 *      and a spread of amax significands -- x any bf16 (subnormals
 *      included), amax >= |x|, s derived
 *      from amax exactly as above -- either q1 == x / s bit for bit, or both
 *      lie below 2^-17 in magnitude with the same sign (every FP8 format
 *      rounds those to a signed zero);
 *  (3) signed zeros.
 * Exit status 0 when every check holds.
 * Build: gcc -O2 -mfma -ffp-contract=off -fno-fast-math
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fb(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bf(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

typedef struct { float s, sp, rp, f; } blk;

static blk block_of(float amax, float M)
{
    blk b;
    volatile float s = amax / M;
    if (s < 0x1p-126f) s = 0x1p-126f;
    b.s = s;
    b.f = amax < 0x1p-60f ? 0x1p64f : 1.0f;
    b.sp = s * b.f;
    b.rp = 1.0f / b.sp;
    return b;
}

/* The GPU code is exactly: e = fma(q0, sp, -x'); q1 = fma(-e, rp, q0).  The
 * volatile keeps gcc from rewriting -fma(a, b, -c) as fnmadd(a, b, c), which
 * differs from it in the sign of a zero result. */
static float kernel_quotient(float x, const blk *b)
{
    float xp = x * b->f;
    float q0 = xp * b->rp;
    volatile float e = fmaf(q0, b->sp, -xp);
    return fmaf(-e, b->rp, q0);
}

static long bad = 0;

static void check(float x, float amax, float M)
{
    blk b = block_of(amax, M);
    float q1 = kernel_quotient(x, &b);
    float q = x / b.s;
    if (bf(q1) == bf(q)) return;
    if (fabsf(q1) < 0x1p-17f && fabsf(q) < 0x1p-17f && signbit(q1) == signbit(q)) return;
    if (bad++ < 10)
        fprintf(stderr, "mismatch x=%a amax=%a M=%g: kernel %a, divide %a\n", x, amax, M, q1, q);
}

int main(void)
{
    /* (1) every significand pair: x in [1,2) with 7 fraction bits, s in [1,2) */
    for (uint32_t xm = 0; xm < 128; ++xm) {
        float x = fb(0x3F800000u | (xm << 16));
        for (uint32_t sm = 0; sm < (1u << 23); ++sm) {
            blk b;
            b.s = fb(0x3F800000u | sm);
            b.f = 1.0f;
            b.sp = b.s;
            b.rp = 1.0f / b.sp;
            float q1 = kernel_quotient(x, &b);
            float q = x / b.s;
            if (bf(q1) != bf(q) && bad++ < 10)
                fprintf(stderr, "pair mismatch x=%a s=%a: %a vs %a\n", x, b.s, q1, q);
        }
    }
    /* (2) exponent grid: every bf16 exponent for x and amax, a spread of
     * significands, both formats, both signs of x */
    const float Ms[2] = {448.0f, 57344.0f};
    const uint32_t sig[] = {0, 1, 2, 0x3F, 0x40, 0x41, 0x55, 0x7E, 0x7F};
    const int nsig = sizeof sig / sizeof sig[0];
    for (int m = 0; m < 2; ++m)
        for (uint32_t ea = 0; ea < 255; ++ea)
            for (int ia = 0; ia < nsig; ++ia) {
                uint32_t abits = (ea << 7) | sig[ia];
                if (abits == 0) continue;
                float amax = fb(abits << 16);
                for (uint32_t ex = 0; ex <= ea; ++ex)
                    for (uint32_t xm = 0; xm < 128; ++xm) {
                        uint32_t xbits = (ex << 7) | xm;
                        if (xbits > abits) continue;
                        float x = fb(xbits << 16);
                        check(x, amax, Ms[m]);
                        check(-x, amax, Ms[m]);
                    }
            }
    /* (3) signed zeros, in a normal block and a zero block */
    for (int m = 0; m < 2; ++m) {
        float amaxes[3] = {0.0f, 1.0f, 0x1p-100f};
        for (int i = 0; i < 3; ++i) {
            blk b = block_of(amaxes[i], Ms[m]);
            float pz = kernel_quotient(0.0f, &b), nz = kernel_quotient(-0.0f, &b);
            if (bf(pz) != 0u || bf(nz) != 0x80000000u) {
                ++bad;
                fprintf(stderr, "signed zero lost: %a %a\n", pz, nz);
            }
        }
    }
    printf("mismatches: %ld\n", bad);
    return bad == 0 ? 0 : 1;
}
