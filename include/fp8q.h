/*
 * fp8q.h -- C ABI of the MI355X (gfx950) FP8 wire codec.
 *
 * The codec is the data-parallel hot path of sending bf16 gradients and
 * weights as FP8 with blockwise scales, and of summing the peers' FP8 chunks
 * on the receiver:
 *   - "FP8 Transmission Optimization for VLA Training: Byte Reduction Leads to
 *     Increased Latency", section "FP8 Transmission Optimization and
 *     Bottlenecks", bullet "Transmission Efficiency": FP8 (e4m3/e5m2) with
 *     blockwise scaling on the wire, and a fused dequantize-then-reduce that
 *     avoids the HBM traffic of dequantizing first and summing after;
 *   - "perf: Reduce MXFP8 refit weight-transfer overheads" (NVIDIA-NeMo/RL
 *     pull request 3294), sections "Summary" and "Safety", and the review's
 *     "Verified clean" list: trainer weights prequantized to E4M3 with an
 *     E8M0 scale per 32 elements, shaped [rows, K/32].
 * The FP8 formats are the OCP ones (OFP8 rev 1.0); E8M0 is the OCP MX v1.0
 * scale type.
 *
 * Conventions shared by every entry point
 *   - Data pointers are DEVICE pointers.  Arrays of pointers (the peers of
 *     fp8q_dequant_reduce, fp8q_dequant_reduce_requantize,
 *     mx8_dequant_reduce and fp8q_sum_f32) are HOST arrays of device
 *     pointers, read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream) of the current
 *     HIP device, and every buffer must live on that device.  Work is
 *     enqueued on it and the call returns without synchronising.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after returning and holds no mutable global state.
 *   - Every argument is checked on the host before anything is launched.  On
 *     any error the call returns a non-zero status, launches nothing and
 *     writes no output byte.  n == 0 (or rows * K == 0) is a successful no-op.
 *   - Bulk data pointers (bf16 inputs, FP8 codes, outputs) must be 16-byte
 *     aligned; fp32 scale arrays 4-byte aligned; E8M0 arrays any alignment.
 *   - No output range may overlap an input range or another output range.
 *   - Element counts are limited to FP8Q_MAX_ELEMS.
 *   - Calls on different streams may run concurrently; the library is
 *     thread-safe.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the ABI; everything else in the library is hidden. */
#if defined(__GNUC__) || defined(__clang__)
#define FP8Q_API __attribute__((visibility("default")))
#else
#define FP8Q_API
#endif

#define FP8Q_ABI_VERSION 1
#define FP8Q_BLOCK 128            /* elements per fp32 scale (block quantize) */
#define FP8Q_MX_BLOCK 32          /* elements per E8M0 scale, along K          */
#define FP8Q_MAX_PEERS 16         /* largest k for fp8q_dequant_reduce         */
#define FP8Q_MAX_ELEMS (((size_t)1) << 40)

typedef enum {
    FP8Q_E4M3 = 0,                /* OCP E4M3: bias 7, max 448, no inf          */
    FP8Q_E5M2 = 1                 /* OCP E5M2: bias 15, max 57344               */
} fp8q_format;

typedef enum {
    FP8Q_OUT_F32 = 0,             /* fp32 output                                */
    FP8Q_OUT_BF16 = 1             /* bf16 output: the fp32 result rounded RNE   */
} fp8q_out_dtype;

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_NULL = 1,            /* a required pointer is NULL                 */
    FP8Q_ERR_ARG = 2,             /* bad enum, k out of range, K % 32 != 0,
                                     or a size above FP8Q_MAX_ELEMS            */
    FP8Q_ERR_ALIGN = 3,           /* a pointer breaks the alignment rule        */
    FP8Q_ERR_OVERLAP = 4,         /* an output overlaps an input or an output   */
    FP8Q_ERR_HIP = 5              /* the HIP runtime reported an error when the
                                     kernels were enqueued (hipGetLastError,
                                     which also returns, and clears, an error
                                     left by earlier work in the thread)        */
} fp8q_status;

/*
 * Block-128 quantize of a flat bf16 tensor ("Transmission Efficiency" bullet:
 * FP8 with blockwise scaling).  For each block b of 128 contiguous elements
 * (the last block may be partial and then covers only the valid elements):
 *   amax_b = max |x_i|
 *   s_b    = max(fl32(amax_b / FP8_MAX), 2^-126)     FP8_MAX = 448 | 57344
 *   q_i    = satRNE_fmt(fl32(x_i / s_b))  (round to nearest even, saturating,
 *                                          signed zero kept)
 * A block holding an inf or NaN gets s_b = NaN (0x7FC00000) and all codes 0x7F.
 *   x_bf16     [n] bf16, device, 16-byte aligned
 *   q_out      [n] uint8 FP8 codes, same order as x, device, 16-byte aligned
 *   scales_out [ceil(n / 128)] fp32, device, 4-byte aligned
 */
FP8Q_API fp8q_status fp8q_quantize(const void *x_bf16, size_t n, fp8q_format fmt,
                          void *q_out, float *scales_out, void *stream);

/*
 * Dequantize one shard: y_i = fl32(dec(q_i) * s_{floor(i/128)}), written as
 * fp32 or as bf16 (RNE of that fp32).
 *   q          [n] uint8, device, 16-byte aligned
 *   scales     [ceil(n / 128)] fp32, device, 4-byte aligned
 *   y_out      [n] fp32 or bf16, device, 16-byte aligned
 */
FP8Q_API fp8q_status fp8q_dequantize(const void *q, const float *scales, size_t n,
                            fp8q_format fmt, void *y_out, fp8q_out_dtype out_dtype,
                            void *stream);

/*
 * Fused dequantize-then-reduce of k peer shards ("Transmission Efficiency"
 * bullet: the fused kernel that removes the naive path's HBM traffic).  No
 * dequantized copy is written to HBM:
 *   d_{p,i} = fl32(dec(q_p[i]) * s_p[floor(i/128)])
 *   acc_i   = d_{0,i};  acc_i = fl32(acc_i + d_{p,i}) for p = 1 .. k-1
 *   y_i     = acc_i (fp32) or RNE_bf16(acc_i)
 * The peers are summed in ascending order, each addition rounded to fp32
 * (no fused multiply-add), so the result is deterministic.
 *   q_peers      host array of k device pointers, each [n] uint8, 16-byte aligned
 *   scales_peers host array of k device pointers, each [ceil(n/128)] fp32
 *   k            1 .. FP8Q_MAX_PEERS
 *   y_out        [n] fp32 or bf16, device, 16-byte aligned
 */
FP8Q_API fp8q_status fp8q_dequant_reduce(const void *const *q_peers, const float *const *scales_peers,
                                int k, size_t n, fp8q_format fmt, void *y_out,
                                fp8q_out_dtype out_dtype, void *stream);

/*
 * MXFP8 weight quantize ("perf: Reduce MXFP8 refit weight-transfer
 * overheads": E4M3 weights with a matching E8M0 scale per 32 elements along
 * K, scales shaped [rows, K/32] even when K == 32).  A 3-D [E, N, K] tensor is
 * passed as rows = E * N.  Per block of 32 contiguous elements along K:
 *   X    = clamp(floor(log2 amax) - 8, -127, 127)       (8 = E4M3's emax)
 *   code = X + 127            (E8M0: 2^(code-127); zero amax -> code 0,
 *                              the zero-scale clamp)
 *   q_i  = satRNE_e4m3(x_i * 2^-X)
 * A block holding an inf or NaN gets code 0xFF and all element codes 0x7F.
 *   w_bf16   [rows, K] bf16 row-major, device, 16-byte aligned
 *   K        a multiple of 32
 *   q_out    [rows, K] uint8 E4M3 codes, device, 16-byte aligned
 *   e8m0_out [rows, K/32] uint8, device
 */
FP8Q_API fp8q_status mx8_quantize(const void *w_bf16, size_t rows, size_t K, void *q_out,
                         void *e8m0_out, void *stream);

/*
 * The second half of the naive dequantize-then-reduce that the fused kernel
 * replaces ("Transmission Efficiency" bullet): sums k fp32 arrays in
 * ascending order, y_i = ((p_0[i] + p_1[i]) + ...) rounded to fp32 at every
 * step, written as fp32 or bf16.  With k fp8q_dequantize calls into fp32
 * buffers first, it gives exactly the fused kernel's result; it exists to
 * measure what the fusion saves.
 *   parts   host array of k device pointers, each [n] fp32, 16-byte aligned
 *   k       1 .. FP8Q_MAX_PEERS
 *   y_out   [n] fp32 or bf16, device, 16-byte aligned
 */
FP8Q_API fp8q_status fp8q_sum_f32(const float *const *parts, int k, size_t n, void *y_out,
                         fp8q_out_dtype out_dtype, void *stream);

/*
 * Fused dequant-reduce, then requantize: the reduced chunk leaves as FP8 again
 * for the all-gather half of an FP8 all-reduce ("FP8 Transmission
 * Optimization for VLA Training", "Threshold Changes" bullet: the FP8
 * AllGather).  The fp32 sums acc_i of fp8q_dequant_reduce (format fmt_in)
 * are block-128 quantized directly into fmt_out, by the rule of
 * fp8q_quantize applied to fp32 values:
 *   s_b = max(fl32(amax_b / FP8_MAX_out), 2^-126),  q_i = satRNE(fl32(acc_i / s_b))
 * A block whose sums hold an inf or NaN gets s_b = NaN and all codes 0x7F.
 *   q_peers, scales_peers, k   as fp8q_dequant_reduce
 *   q_out      [n] uint8, device, 16-byte aligned
 *   scales_out [ceil(n / 128)] fp32, device, 4-byte aligned
 * The outputs may overlap neither each other nor any peer's input.
 */
FP8Q_API fp8q_status fp8q_dequant_reduce_requantize(const void *const *q_peers,
                                                    const float *const *scales_peers, int k,
                                                    size_t n, fp8q_format fmt_in,
                                                    fp8q_format fmt_out, void *q_out,
                                                    float *scales_out, void *stream);

/*
 * MXFP8 receiver side ("perf: Reduce MXFP8 refit weight-transfer overheads":
 * the receiver of the prequantized weights, whose E8M0 zero-scale clamp must
 * agree with the trainer's -- review "Verified clean").  Per element of the
 * [rows, K] codes, with the [rows, K/32] E8M0 bytes of mx8_quantize:
 *   d = dec_e4m3(q) * 2^(code - 127)      (exact in fp32 unless it overflows
 *                                          to +-inf; code 0xFF -> NaN)
 * mx8_dequant_reduce sums k such shards in peer order, each addition rounded
 * to fp32; mx8_dequantize is k = 1.  Output fp32, or bf16 (RNE of the fp32).
 *   q / q_peers        [rows, K] uint8 E4M3 codes, device, 16-byte aligned
 *   e8m0 / e8m0_peers  [rows, K/32] uint8, device, any alignment
 *   K                  a multiple of 32;   k   1 .. FP8Q_MAX_PEERS
 *   y_out              [rows, K] fp32 or bf16, device, 16-byte aligned
 */
FP8Q_API fp8q_status mx8_dequantize(const void *q, const void *e8m0, size_t rows, size_t K,
                                    void *y_out, fp8q_out_dtype out_dtype, void *stream);
FP8Q_API fp8q_status mx8_dequant_reduce(const void *const *q_peers, const void *const *e8m0_peers,
                                        int k, size_t rows, size_t K, void *y_out,
                                        fp8q_out_dtype out_dtype, void *stream);

/*
 * Tensorwise quantize: one fp32 scale for the whole tensor, the tensorwise
 * recipe (amax, scale and cast per tensor) named on "How to Speed Up VLA
 * Training Step by Step: A 3x Acceleration Case Study on Pi0.5", FP8 section.
 * The rule of fp8q_quantize with one block spanning the tensor:
 *   s = max(fl32(amax / FP8_MAX), 2^-126),  q_i = satRNE(fl32(x_i / s))
 * (inf or NaN anywhere: s = NaN, all codes 0x7F).  The input is read twice
 * (an amax pass, then the quantize pass).  *scale_out is also the amax slot
 * while the call's kernels run: it holds the scale once they have finished.
 *   x_bf16     [n] bf16, device, 16-byte aligned
 *   q_out      [n] uint8, device, 16-byte aligned
 *   scale_out  one fp32, device, 4-byte aligned
 */
FP8Q_API fp8q_status fp8q_quantize_tensorwise(const void *x_bf16, size_t n, fp8q_format fmt,
                                              void *q_out, float *scale_out, void *stream);

/* A static, human-readable name for a status code (never NULL). */
FP8Q_API const char *fp8q_status_str(fp8q_status s);

/* FP8Q_ABI_VERSION of the built library. */
FP8Q_API int fp8q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
