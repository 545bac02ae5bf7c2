/*
 * fp8q_oracle.c -- plain, slow CPU oracle for the FP8 wire codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library, and it defines the results the HIP library must reproduce.
 *
 * Sources (the method).  The pages this follows:
 *   [VLA-FP8]  "FP8 Transmission Optimization for VLA Training: Byte Reduction
 *              Leads to Increased Latency", section "FP8 Transmission
 *              Optimization and Bottlenecks", bullet "Transmission Efficiency":
 *              bf16 DP gradients are sent as FP8 (e4m3 or e5m2) with blockwise
 *              scaling, and the receiver sums the peers' FP8 chunks with a fused
 *              dequantize-then-reduce.
 *   [MXFP8-PR] "perf: Reduce MXFP8 refit weight-transfer overheads"
 *              (NVIDIA-NeMo/RL pull request 3294): sections "Summary" and
 *              "Safety" (trainer weights prequantized to E4M3 with a matching
 *              per-block scale tensor), the self-review's "Verified clean"
 *              list (E8M0 zero-scale clamp, scales of shape [M, K/32]), and the
 *              inline review "[Minor, latent] Unconditional squeeze(dim=-1)"
 *              (the K/32 scale dimension is real even when it is 1).
 * Sources (the formats).  The pages name e4m3, e5m2 and E8M0 without defining
 * them; the definitions are the public OCP specifications:
 *   OCP 8-bit Floating Point Specification (OFP8), rev. 1.0, tables of the
 *   E4M3 and E5M2 encodings; OCP Microscaling Formats (MX) Specification v1.0,
 *   the E8M0 scale type and the MX scale-selection rule.
 *
 * Where the pages leave a step open the plainest reading is taken; each such
 * reading is marked READING below.  One function, the tensorwise quantize,
 * follows a recipe the pages name without printing its arithmetic: its
 * parity against that recipe is unpinned (marked PARITY UNPINNED below).
 *
 * Precision.  The method fixes its own arithmetic: an fp32 scale per block,
 * an fp32 quotient that is then rounded to FP8, and fp32 accumulation.  So
 * this oracle computes in fp32 exactly where the method does; the FP8 rounding
 * itself is done exactly in double (every value involved is a double).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * FP contraction must stay off: every fp32 operation here is rounded alone.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_E4M3 0
#define ORACLE_E5M2 1

/* ------------------------------------------------------------------------ */
/* bit helpers                                                               */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t b)
{
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f)
{
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* bf16 is the top half of an fp32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    return f32_from_bits((uint32_t)h << 16);
}

/* fp32 -> bf16, round to nearest, ties to even; overflow gives +-inf.
 * READING: a NaN input gives the canonical quiet NaN 0x7FC0. */
uint16_t oracle_f32_to_bf16(float f)
{
    if (isnan(f))
        return 0x7FC0;
    uint32_t b = bits_from_f32(f);
    uint32_t lsb = (b >> 16) & 1u;          /* ties go to the even result */
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 format parameters (OFP8 rev 1.0)                                  */
/*   E4M3: 4 exponent bits, bias 7, 3 mantissa bits, no infinities,          */
/*         S.1111.111 is NaN, largest finite S.1111.110 = 448.               */
/*   E5M2: 5 exponent bits, bias 15, 2 mantissa bits, IEEE-like:             */
/*         S.11111.00 is inf, S.11111.{01,10,11} NaN, largest finite 57344.  */
/* ------------------------------------------------------------------------ */

static int fmt_mbits(int fmt) { return fmt == ORACLE_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == ORACLE_E4M3 ? 7 : 15; }
static uint8_t fmt_max_code(int fmt) { return fmt == ORACLE_E4M3 ? 0x7E : 0x7B; }

/* Largest finite value of the format (448 or 57344), in the format's own terms. */
double oracle_fp8_max(int fmt)
{
    return fmt == ORACLE_E4M3 ? 448.0 : 57344.0;
}

/* Decode one FP8 code to its exact value (every FP8 value is an fp32). */
float oracle_fp8_decode(uint8_t code, int fmt)
{
    const int mbits = fmt_mbits(fmt);
    const int ebits = 7 - mbits;
    const int bias = fmt_bias(fmt);
    const int sign = code >> 7;
    const int E = (code >> mbits) & ((1 << ebits) - 1);
    const int M = code & ((1 << mbits) - 1);
    const int emax_field = (1 << ebits) - 1;
    double v;

    if (fmt == ORACLE_E4M3 && E == emax_field && M == (1 << mbits) - 1)
        return NAN;                                    /* S.1111.111 */
    if (fmt == ORACLE_E5M2 && E == emax_field)
        return M == 0 ? (sign ? -INFINITY : INFINITY) : NAN;

    if (E == 0)            /* subnormal: 2^(1-bias) * M / 2^mbits */
        v = ldexp((double)M, 1 - bias - mbits);
    else                   /* normal: 2^(E-bias) * (1 + M / 2^mbits) */
        v = ldexp(1.0 + (double)M / (double)(1 << mbits), E - bias);
    return (float)(sign ? -v : v);
}

/*
 * satRNE: round a real value y (given exactly as a double) to the FP8 format,
 * to nearest with ties to the even code, saturating to the largest finite
 * magnitude instead of overflowing.  Signed zero is kept (-0 -> 0x80).
 * READING: NaN -> 0x7F (canonical NaN, sign cleared); +-inf saturates like any
 * other overflow.  E5M2 therefore never emits an infinity code.
 */
uint8_t oracle_fp8_encode(double y, int fmt)
{
    const int mbits = fmt_mbits(fmt);
    const int bias = fmt_bias(fmt);
    const int emin = 1 - bias;                 /* exponent of the min normal */
    const double maxv = oracle_fp8_max(fmt);
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a, quantum, m, r;
    int ex, u;

    if (isnan(y))
        return 0x7F;
    a = fabs(y);
    if (a == 0.0)
        return sign;
    if (isinf(a) || a >= 2.0 * maxv)           /* far beyond the range */
        return sign | fmt_max_code(fmt);

    /* Representable magnitudes near a are multiples of 2^(max(u, emin) - mbits)
     * where u = floor(log2 a). */
    (void)frexp(a, &ex);                        /* a = f * 2^ex, f in [0.5, 1) */
    u = ex - 1;
    quantum = ldexp(1.0, (u > emin ? u : emin) - mbits);
    m = nearbyint(a / quantum);                 /* exact quotient; RNE (default mode) */
    r = m * quantum;                            /* nearest representable, exact */
    if (r > maxv)
        return sign | fmt_max_code(fmt);        /* saturate */
    if (r == 0.0)
        return sign;

    /* encode the representable value r */
    if (r < ldexp(1.0, emin)) {                 /* subnormal: E = 0, M = r / 2^(emin-mbits) */
        int M = (int)(r / ldexp(1.0, emin - mbits));
        return sign | (uint8_t)M;
    } else {
        int E, M;
        (void)frexp(r, &ex);
        u = ex - 1;                             /* may be one more than before after rounding up */
        E = u + bias;
        M = (int)((r / ldexp(1.0, u) - 1.0) * (double)(1 << mbits));
        return sign | (uint8_t)((E << mbits) | M);
    }
}

/* ------------------------------------------------------------------------ */
/* Block-128 quantize [VLA-FP8, Transmission Efficiency]                    */
/*                                                                          */
/* For block b = elements [128b, min(128b+128, n)):                          */
/*   amax_b = max |x_i| over the block's valid elements;                     */
/*   s_b    = max(fl32(amax_b / FP8_MAX), 2^-126)                            */
/*   q_i    = satRNE(fl32(x_i / s_b))                                        */
/* READING: scale = block amax / the format's largest finite value, stored   */
/* as fp32; the element is divided by that stored scale.  A block whose      */
/* amax is zero (or tiny) gets the smallest normal fp32 scale 2^-126, the    */
/* counterpart of the zero-scale clamp of [MXFP8-PR, Verified clean].        */
/* READING: a block holding an inf or NaN gets scale NaN (0x7FC00000) and    */
/* every code 0x7F.                                                          */
/* ------------------------------------------------------------------------ */

#define ORACLE_BLOCK 128

/* Element accessors: the block step reads bf16 inputs (widened exactly) or
 * fp32 inputs (the requantize of a reduced sum). */
static float elem_bf16(const void *p, size_t i) { return oracle_bf16_to_f32(((const uint16_t *)p)[i]); }
static float elem_f32(const void *p, size_t i) { return ((const float *)p)[i]; }

/* One block of `len` values: amax, scale, codes. */
static void quantize_block_any(const void *x, float (*elem)(const void *, size_t), size_t len,
                               int fmt, uint8_t *q, float *scale)
{
    const float fmax = (float)oracle_fp8_max(fmt);
    const float smin = ldexpf(1.0f, -126);
    float amax = 0.0f, s;
    size_t i;

    for (i = 0; i < len; ++i) {
        float v = elem(x, i);
        if (!isfinite(v)) {
            *scale = f32_from_bits(0x7FC00000u);
            for (i = 0; i < len; ++i)
                q[i] = 0x7F;
            return;
        }
        if (fabsf(v) > amax)
            amax = fabsf(v);
    }
    s = amax / fmax;                 /* IEEE fp32 divide */
    if (s < smin)
        s = smin;
    *scale = s;
    for (i = 0; i < len; ++i) {
        float qf = elem(x, i) / s;   /* fp32 quotient, rounded once */
        q[i] = oracle_fp8_encode((double)qf, fmt);
    }
}

void oracle_quantize_block(const uint16_t *x, size_t len, int fmt,
                           uint8_t *q, float *scale)
{
    quantize_block_any(x, elem_bf16, len, fmt, q, scale);
}

void oracle_quantize(const uint16_t *x, size_t n, int fmt, uint8_t *q, float *scales)
{
    size_t b, nb = (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (b = 0; b < nb; ++b) {
        size_t lo = b * ORACLE_BLOCK;
        size_t len = n - lo < ORACLE_BLOCK ? n - lo : ORACLE_BLOCK;
        oracle_quantize_block(x + lo, len, fmt, q + lo, scales + b);
    }
}

/* ------------------------------------------------------------------------ */
/* Tensorwise quantize: one fp32 scale for the whole tensor.                 */
/* The Pi0.5 page ("How to Speed Up VLA Training Step by Step", the FP8      */
/* section on TorchAO's Float8Linear with the tensorwise recipe) computes    */
/* amax, scale and cast per tensor.  READING: the same scale rule and floor  */
/* as the block path, with the block being the whole tensor.                 */
/* PARITY UNPINNED against that recipe: the page names it but prints none of */
/* its arithmetic (its scale formula, rounding or floor), and no library     */
/* implementing it is available here, so this function is pinned only to    */
/* the block rule (one block spanning the tensor equals block quantize).     */
/* ------------------------------------------------------------------------ */

void oracle_quantize_tensorwise(const uint16_t *x, size_t n, int fmt, uint8_t *q, float *scale)
{
    quantize_block_any(x, elem_bf16, n, fmt, q, scale);
}

/* ------------------------------------------------------------------------ */
/* Dequantize one shard: y_i = fl32(dec(q_i) * s_{i/128}).                   */
/* Output as fp32, or as bf16 = RNE_bf16 of that fp32 (out_bf16 != 0).      */
/* ------------------------------------------------------------------------ */

void oracle_dequantize(const uint8_t *q, const float *scales, size_t n, int fmt,
                       void *y, int out_bf16)
{
    size_t i;
    for (i = 0; i < n; ++i) {
        float d = oracle_fp8_decode(q[i], fmt) * scales[i / ORACLE_BLOCK];
        if (out_bf16)
            ((uint16_t *)y)[i] = oracle_f32_to_bf16(d);
        else
            ((float *)y)[i] = d;
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantize-then-reduce of k peer shards [VLA-FP8, Transmission            */
/* Efficiency: the receiver's fused dequantize-then-reduce].                 */
/*   d_{p,i} = fl32(dec(q_p[i]) * s_p[i/128])                                */
/*   acc = d_{0,i};  acc = fl32(acc + d_{p,i}) for p = 1 .. k-1              */
/* READING: the sum runs over peers in ascending order, each step rounded    */
/* to fp32, starting from peer 0's value (so k = 1 is exactly a dequantize,  */
/* -0 included).  The output is acc (fp32) or RNE_bf16(acc).                 */
/* ------------------------------------------------------------------------ */

/* acc over the k peers for element i */
static float reduce_one(const uint8_t *const *q, const float *const *scales, int k, size_t i, int fmt)
{
    float acc = oracle_fp8_decode(q[0][i], fmt) * scales[0][i / ORACLE_BLOCK];
    int p;
    for (p = 1; p < k; ++p) {
        float d = oracle_fp8_decode(q[p][i], fmt) * scales[p][i / ORACLE_BLOCK];
        acc = acc + d;
    }
    return acc;
}

void oracle_dequant_reduce(const uint8_t *const *q, const float *const *scales, int k,
                           size_t n, int fmt, void *y, int out_bf16)
{
    size_t i;
    for (i = 0; i < n; ++i) {
        float acc = reduce_one(q, scales, k, i, fmt);
        if (out_bf16)
            ((uint16_t *)y)[i] = oracle_f32_to_bf16(acc);
        else
            ((float *)y)[i] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantize-reduce, then requantize the reduced chunk: the step after the  */
/* fused reduce in an FP8 all-reduce, whose all-gather half sends FP8 again  */
/* ("FP8 Transmission Optimization for VLA Training", "Threshold Changes":   */
/* the FP8 AllGather).  READING: the reduced fp32 values are block-128       */
/* quantized directly (no bf16 rounding in between), by the same block step  */
/* as the bf16 path, into the output format.                                 */
/* ------------------------------------------------------------------------ */

void oracle_reduce_requantize(const uint8_t *const *q, const float *const *scales, int k,
                              size_t n, int fmt_in, int fmt_out, uint8_t *q_out, float *s_out)
{
    float acc[ORACLE_BLOCK];
    size_t b, j, nb = (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (b = 0; b < nb; ++b) {
        size_t lo = b * ORACLE_BLOCK;
        size_t len = n - lo < ORACLE_BLOCK ? n - lo : ORACLE_BLOCK;
        for (j = 0; j < len; ++j)
            acc[j] = reduce_one(q, scales, k, lo + j, fmt_in);
        quantize_block_any(acc, elem_f32, len, fmt_out, q_out + lo, s_out + b);
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 weight quantize [MXFP8-PR, Summary / Safety / Verified clean].      */
/* Weights [rows, K] row-major (a 3-D [E, N, K] tensor is rows = E*N); one   */
/* E8M0 scale per 32 contiguous elements along K, stored as [rows, K/32].    */
/*   X    = clamp(floor(log2 amax) - 8, -127, 127)    (8 = E4M3's emax)      */
/*   code = X + 127                 (E8M0: value 2^(code-127); 0xFF is NaN)   */
/*   q_i  = satRNE_e4m3(x_i * 2^-X)                                          */
/* amax == 0 gives X = -127, code 0: the "zero-scale clamp".                 */
/* READING: the scale rule is the OCP MX v1.0 one (the pages do not print    */
/* it); a block holding inf or NaN gets code 0xFF and every element 0x7F.    */
/* ------------------------------------------------------------------------ */

#define ORACLE_MX_BLOCK 32

void oracle_mx8_quantize_block(const uint16_t *w, uint8_t *q, uint8_t *e8m0)
{
    float amax = 0.0f;
    int i, X, ex;

    for (i = 0; i < ORACLE_MX_BLOCK; ++i) {
        float v = oracle_bf16_to_f32(w[i]);
        if (!isfinite(v)) {
            *e8m0 = 0xFF;
            for (i = 0; i < ORACLE_MX_BLOCK; ++i)
                q[i] = 0x7F;
            return;
        }
        if (fabsf(v) > amax)
            amax = fabsf(v);
    }
    if (amax == 0.0f) {
        X = -127;
    } else {
        (void)frexpf(amax, &ex);               /* amax = f * 2^ex, f in [0.5, 1) */
        X = (ex - 1) - 8;                       /* floor(log2 amax) - emax(E4M3) */
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    *e8m0 = (uint8_t)(X + 127);
    for (i = 0; i < ORACLE_MX_BLOCK; ++i) {
        double v = ldexp((double)oracle_bf16_to_f32(w[i]), -X);   /* exact */
        q[i] = oracle_fp8_encode(v, ORACLE_E4M3);
    }
}

/* returns 0 on success, -1 if K is not a multiple of 32 */
int oracle_mx8_quantize(const uint16_t *w, size_t rows, size_t K, uint8_t *q, uint8_t *e8m0)
{
    size_t r, j, nbk;
    if (K % ORACLE_MX_BLOCK != 0)
        return -1;
    nbk = K / ORACLE_MX_BLOCK;
    for (r = 0; r < rows; ++r)
        for (j = 0; j < nbk; ++j)
            oracle_mx8_quantize_block(w + r * K + j * ORACLE_MX_BLOCK,
                                      q + r * K + j * ORACLE_MX_BLOCK,
                                      e8m0 + r * nbk + j);
    return 0;
}

/* Decode an E8M0 scale code to its value 2^(code-127); 0xFF is NaN. */
float oracle_e8m0_decode(uint8_t code)
{
    if (code == 0xFF)
        return NAN;
    return ldexpf(1.0f, (int)code - 127);
}

/* ------------------------------------------------------------------------ */
/* MXFP8 receiver side: y = dec_e4m3(q) * 2^(code-127) per 32 along K, and   */
/* the k-peer ordered fp32 sum of such values.  The pages check that the     */
/* trainer's and the receiver's E8M0 zero-scale clamp agree ("perf: Reduce   */
/* MXFP8 refit weight-transfer overheads", self-review, "Verified clean").   */
/* The product is exact in fp32 (a 4-bit significand times a power of two   */
/* no smaller than 2^-127) unless it overflows to +-inf, which codes made by */
/* mx8_quantize never do.  READING: output fp32, or bf16 = RNE of it.        */
/* ------------------------------------------------------------------------ */

static float mx_value(const uint8_t *q, const uint8_t *e8m0, size_t K, size_t r, size_t c)
{
    return oracle_fp8_decode(q[r * K + c], ORACLE_E4M3) *
           oracle_e8m0_decode(e8m0[r * (K / ORACLE_MX_BLOCK) + c / ORACLE_MX_BLOCK]);
}

int oracle_mx8_dequant_reduce(const uint8_t *const *q, const uint8_t *const *e8m0, int k,
                              size_t rows, size_t K, void *y, int out_bf16)
{
    size_t r, c;
    int p;
    if (K % ORACLE_MX_BLOCK != 0)
        return -1;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < K; ++c) {
            float acc = mx_value(q[0], e8m0[0], K, r, c);
            for (p = 1; p < k; ++p) {
                float d = mx_value(q[p], e8m0[p], K, r, c);
                acc = acc + d;
            }
            if (out_bf16)
                ((uint16_t *)y)[r * K + c] = oracle_f32_to_bf16(acc);
            else
                ((float *)y)[r * K + c] = acc;
        }
    return 0;
}

int oracle_mx8_dequantize(const uint8_t *q, const uint8_t *e8m0, size_t rows, size_t K,
                          void *y, int out_bf16)
{
    return oracle_mx8_dequant_reduce(&q, &e8m0, 1, rows, K, y, out_bf16);
}

/* Vectorised converter entry points, for exhaustive tests. */
void oracle_fp8_encode_f32_array(const float *y, size_t n, int fmt, uint8_t *out)
{
    size_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_fp8_encode((double)y[i], fmt);
}

void oracle_fp8_decode_array(const uint8_t *c, size_t n, int fmt, float *out)
{
    size_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_fp8_decode(c[i], fmt);
}
