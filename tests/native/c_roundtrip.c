/*
 * A C caller of libfp8q with no Python and no torch: device buffers from
 * hipMalloc, a stream from hipStreamCreate, host arrays of peer pointers.
 * Runs block quantize (e4m3, e5m2), the fused dequant-reduce of 3 peers
 * (fp32 and bf16 out), the requantize, MXFP8 quantize and the MXFP8
 * receiver, and checks every output byte against the C oracle
 * (oracle/liboracle.so) on the same inputs.  Also checks that a rejected
 * call returns its status and leaves its output untouched.
 * Exit status 0 and "c_roundtrip ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp8q.h"

/* the oracle's C entry points (oracle/fp8q_oracle.c) */
void oracle_quantize(const uint16_t *x, size_t n, int fmt, uint8_t *q, float *scales);
void oracle_dequant_reduce(const uint8_t *const *q, const float *const *scales, int k,
                           size_t n, int fmt, void *y, int out_bf16);
void oracle_reduce_requantize(const uint8_t *const *q, const float *const *scales, int k,
                              size_t n, int fmt_in, int fmt_out, uint8_t *q_out, float *s_out);
int oracle_mx8_quantize(const uint16_t *w, size_t rows, size_t K, uint8_t *q, uint8_t *e8m0);
int oracle_mx8_dequant_reduce(const uint8_t *const *q, const uint8_t *const *e8m0, int k,
                              size_t rows, size_t K, void *y, int out_bf16);

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));  \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)
#define CHECK_FP8Q(x)                                                             \
  do {                                                                            \
    fp8q_status s_ = (x);                                                         \
    if (s_ != FP8Q_OK) {                                                          \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, fp8q_status_str(s_));    \
      exit(3);                                                                    \
    }                                                                             \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}

/* finite bf16 values of assorted magnitudes, some zeros */
static uint16_t random_bf16(void) {
  uint64_t r = next_u64();
  uint16_t sign = (uint16_t)((r >> 63) << 15);
  uint16_t exp = (uint16_t)(100 + (r >> 32) % 40);      /* about 2^-27 .. 2^12 */
  uint16_t man = (uint16_t)(r & 0x7F);
  if ((r >> 40) % 97 == 0) return sign;                /* signed zero */
  return (uint16_t)(sign | (exp << 7) | man);
}

static void *dev_copy(const void *h, size_t bytes) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static int same(const void *a, const void *b, size_t bytes, const char *what) {
  if (memcmp(a, b, bytes) != 0) {
    const uint8_t *x = a, *y = b;
    size_t i = 0;
    while (x[i] == y[i]) ++i;
    fprintf(stderr, "%s differs at byte %zu (%02x vs %02x)\n", what, i, x[i], y[i]);
    return 0;
  }
  return 1;
}

int main(void) {
  enum { K_PEERS = 3 };
  const size_t n = 128 * 5000 + 77;                   /* many tiles and a ragged tail */
  const size_t nb = (n + 127) / 128;
  const size_t rows = 96, K = 2048;                    /* MXFP8 weights */
  int ok = 1;
  hipStream_t st;
  CHECK_HIP(hipStreamCreate(&st));

  uint16_t *x[K_PEERS];
  for (int p = 0; p < K_PEERS; ++p) {
    x[p] = malloc(n * 2);
    for (size_t i = 0; i < n; ++i) x[p][i] = random_bf16();
  }
  for (int fmt = 0; fmt < 2; ++fmt) {
    uint8_t *qh[K_PEERS], *qo[K_PEERS];
    float *sh[K_PEERS], *so[K_PEERS];
    void *qd[K_PEERS], *sd[K_PEERS];
    for (int p = 0; p < K_PEERS; ++p) {
      void *xd = dev_copy(x[p], n * 2);
      CHECK_HIP(hipMalloc(&qd[p], n));
      CHECK_HIP(hipMalloc(&sd[p], nb * 4));
      CHECK_FP8Q(fp8q_quantize(xd, n, (fp8q_format)fmt, qd[p], (float *)sd[p], st));
      CHECK_HIP(hipStreamSynchronize(st));
      qh[p] = malloc(n); sh[p] = malloc(nb * 4);
      qo[p] = malloc(n); so[p] = malloc(nb * 4);
      CHECK_HIP(hipMemcpy(qh[p], qd[p], n, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(sh[p], sd[p], nb * 4, hipMemcpyDeviceToHost));
      oracle_quantize(x[p], n, fmt, qo[p], so[p]);
      ok &= same(qh[p], qo[p], n, "quantize codes");
      ok &= same(sh[p], so[p], nb * 4, "quantize scales");
      CHECK_HIP(hipFree(xd));
    }
    for (int bf = 0; bf < 2; ++bf) {
      const size_t yb = n * (bf ? 2 : 4);
      void *yd = NULL;
      CHECK_HIP(hipMalloc(&yd, yb));
      CHECK_FP8Q(fp8q_dequant_reduce((const void *const *)qd, (const float *const *)sd, K_PEERS, n,
                                     (fp8q_format)fmt, yd,
                                     bf ? FP8Q_OUT_BF16 : FP8Q_OUT_F32, st));
      CHECK_HIP(hipStreamSynchronize(st));
      void *yh = malloc(yb), *yo = malloc(yb);
      CHECK_HIP(hipMemcpy(yh, yd, yb, hipMemcpyDeviceToHost));
      oracle_dequant_reduce((const uint8_t *const *)qo, (const float *const *)so, K_PEERS, n, fmt,
                            yo, bf);
      ok &= same(yh, yo, yb, bf ? "reduce bf16" : "reduce fp32");
      free(yh); free(yo);
      CHECK_HIP(hipFree(yd));
    }
    {
      void *rq = NULL, *rs = NULL;
      CHECK_HIP(hipMalloc(&rq, n));
      CHECK_HIP(hipMalloc(&rs, nb * 4));
      CHECK_FP8Q(fp8q_dequant_reduce_requantize((const void *const *)qd, (const float *const *)sd,
                                                K_PEERS, n, (fp8q_format)fmt, FP8Q_E4M3, rq,
                                                (float *)rs, st));
      CHECK_HIP(hipStreamSynchronize(st));
      uint8_t *rqh = malloc(n), *rqo = malloc(n);
      float *rsh = malloc(nb * 4), *rso = malloc(nb * 4);
      CHECK_HIP(hipMemcpy(rqh, rq, n, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(rsh, rs, nb * 4, hipMemcpyDeviceToHost));
      oracle_reduce_requantize((const uint8_t *const *)qo, (const float *const *)so, K_PEERS, n,
                               fmt, 0, rqo, rso);
      ok &= same(rqh, rqo, n, "requantize codes");
      ok &= same(rsh, rso, nb * 4, "requantize scales");
      free(rqh); free(rqo); free(rsh); free(rso);
      CHECK_HIP(hipFree(rq)); CHECK_HIP(hipFree(rs));
    }
    /* a rejected call: misaligned output, nothing written */
    {
      uint8_t canary[64], back[64];
      void *yd = NULL;
      memset(canary, 0xC3, sizeof canary);
      CHECK_HIP(hipMalloc(&yd, 64));
      CHECK_HIP(hipMemcpy(yd, canary, 64, hipMemcpyHostToDevice));
      fp8q_status s = fp8q_dequant_reduce((const void *const *)qd, (const float *const *)sd,
                                          K_PEERS, 8, (fp8q_format)fmt, (char *)yd + 4,
                                          FP8Q_OUT_F32, st);
      CHECK_HIP(hipStreamSynchronize(st));
      CHECK_HIP(hipMemcpy(back, yd, 64, hipMemcpyDeviceToHost));
      if (s != FP8Q_ERR_ALIGN) {
        fprintf(stderr, "misaligned output: got status %d\n", (int)s);
        ok = 0;
      }
      ok &= same(back, canary, 64, "rejected call canary");
      CHECK_HIP(hipFree(yd));
    }
    for (int p = 0; p < K_PEERS; ++p) {
      CHECK_HIP(hipFree(qd[p])); CHECK_HIP(hipFree(sd[p]));
      free(qh[p]); free(sh[p]); free(qo[p]); free(so[p]);
    }
  }
  /* MXFP8: quantize 3 peers of weights, then the receiver's reduce */
  {
    const size_t nw = rows * K, ne = nw / 32;
    uint16_t *w = malloc(nw * 2);
    uint8_t *qh[K_PEERS], *eh[K_PEERS], *qo[K_PEERS], *eo[K_PEERS];
    void *qd[K_PEERS], *ed[K_PEERS];
    for (int p = 0; p < K_PEERS; ++p) {
      for (size_t i = 0; i < nw; ++i) w[i] = random_bf16();
      void *wd = dev_copy(w, nw * 2);
      CHECK_HIP(hipMalloc(&qd[p], nw));
      CHECK_HIP(hipMalloc(&ed[p], ne));
      CHECK_FP8Q(mx8_quantize(wd, rows, K, qd[p], ed[p], st));
      CHECK_HIP(hipStreamSynchronize(st));
      qh[p] = malloc(nw); eh[p] = malloc(ne); qo[p] = malloc(nw); eo[p] = malloc(ne);
      CHECK_HIP(hipMemcpy(qh[p], qd[p], nw, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(eh[p], ed[p], ne, hipMemcpyDeviceToHost));
      oracle_mx8_quantize(w, rows, K, qo[p], eo[p]);
      ok &= same(qh[p], qo[p], nw, "mx8 codes");
      ok &= same(eh[p], eo[p], ne, "mx8 e8m0");
      CHECK_HIP(hipFree(wd));
    }
    void *yd = NULL;
    CHECK_HIP(hipMalloc(&yd, nw * 4));
    CHECK_FP8Q(mx8_dequant_reduce((const void *const *)qd, (const void *const *)ed, K_PEERS, rows,
                                  K, yd, FP8Q_OUT_F32, st));
    CHECK_HIP(hipStreamSynchronize(st));
    float *yh = malloc(nw * 4), *yo = malloc(nw * 4);
    CHECK_HIP(hipMemcpy(yh, yd, nw * 4, hipMemcpyDeviceToHost));
    oracle_mx8_dequant_reduce((const uint8_t *const *)qo, (const uint8_t *const *)eo, K_PEERS,
                              rows, K, yo, 0);
    ok &= same(yh, yo, nw * 4, "mx8 reduce");
    free(yh); free(yo); free(w);
    CHECK_HIP(hipFree(yd));
    for (int p = 0; p < K_PEERS; ++p) {
      CHECK_HIP(hipFree(qd[p])); CHECK_HIP(hipFree(ed[p]));
      free(qh[p]); free(eh[p]); free(qo[p]); free(eo[p]);
    }
  }
  for (int p = 0; p < K_PEERS; ++p) free(x[p]);
  CHECK_HIP(hipStreamDestroy(st));
  if (!ok) return 1;
  printf("c_roundtrip ok\n");
  return 0;
}
