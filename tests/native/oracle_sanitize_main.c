/*
 * Drives every oracle entry point on awkward sizes (empty, 1, ragged tails,
 * one block, several blocks, K = 32) so that AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's indexing on the host.
 * Buffers are allocated to their exact sizes, so any overrun is reported.
 * Build: gcc -fsanitize=address,undefined -fno-sanitize-recover=all ...
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_quantize(const uint16_t *x, size_t n, int fmt, uint8_t *q, float *scales);
void oracle_quantize_tensorwise(const uint16_t *x, size_t n, int fmt, uint8_t *q, float *scale);
void oracle_dequantize(const uint8_t *q, const float *scales, size_t n, int fmt, void *y, int bf16);
void oracle_dequant_reduce(const uint8_t *const *q, const float *const *scales, int k, size_t n,
                           int fmt, void *y, int bf16);
void oracle_reduce_requantize(const uint8_t *const *q, const float *const *scales, int k, size_t n,
                              int fmt_in, int fmt_out, uint8_t *q_out, float *s_out);
int oracle_mx8_quantize(const uint16_t *w, size_t rows, size_t K, uint8_t *q, uint8_t *e8m0);
int oracle_mx8_dequant_reduce(const uint8_t *const *q, const uint8_t *const *e8m0, int k,
                              size_t rows, size_t K, void *y, int bf16);

static uint32_t rng = 12345u;
static uint16_t rand16(void)
{
    rng = rng * 1664525u + 1013904223u;
    return (uint16_t)(rng >> 16);
}

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) exit(2); return p; }

int main(void)
{
    const size_t sizes[] = {0, 1, 2, 7, 127, 128, 129, 255, 256, 1000};
    size_t i, j;
    int fmt, k;
    for (i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) {
        size_t n = sizes[i], nb = (n + 127) / 128;
        for (fmt = 0; fmt < 2; ++fmt) {
            uint16_t *x = xmalloc(2 * n);
            uint8_t *q[3];
            float *s[3];
            for (j = 0; j < n; ++j) x[j] = rand16();
            for (k = 0; k < 3; ++k) {
                q[k] = xmalloc(n);
                s[k] = xmalloc(4 * nb);
                oracle_quantize(x, n, fmt, q[k], s[k]);
            }
            {
                float *y = xmalloc(4 * n);
                uint16_t *yb = xmalloc(2 * n);
                uint8_t *qo = xmalloc(n);
                float *so = xmalloc(4 * nb);
                float st;
                oracle_dequantize(q[0], s[0], n, fmt, y, 0);
                oracle_dequantize(q[0], s[0], n, fmt, yb, 1);
                oracle_dequant_reduce((const uint8_t *const *)q, (const float *const *)s, 3, n, fmt, y, 0);
                oracle_dequant_reduce((const uint8_t *const *)q, (const float *const *)s, 3, n, fmt, yb, 1);
                oracle_reduce_requantize((const uint8_t *const *)q, (const float *const *)s, 3, n, fmt,
                                         1 - fmt, qo, so);
                if (n) oracle_quantize_tensorwise(x, n, fmt, qo, &st);
                free(y); free(yb); free(qo); free(so);
            }
            for (k = 0; k < 3; ++k) { free(q[k]); free(s[k]); }
            free(x);
        }
    }
    {
        const size_t shapes[][2] = {{1, 32}, {3, 96}, {5, 64}, {0, 32}, {2, 0}};
        for (i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
            size_t rows = shapes[i][0], K = shapes[i][1], n = rows * K;
            uint16_t *w = xmalloc(2 * n);
            uint8_t *q = xmalloc(n), *e = xmalloc(n / 32);
            float *y = xmalloc(4 * n);
            for (j = 0; j < n; ++j) w[j] = rand16();
            if (oracle_mx8_quantize(w, rows, K, q, e) != 0) return 3;
            {
                const uint8_t *qp[2] = {q, q};
                const uint8_t *ep[2] = {e, e};
                if (oracle_mx8_dequant_reduce(qp, ep, 2, rows, K, y, 0) != 0) return 4;
            }
            free(w); free(q); free(e); free(y);
        }
        {
            uint16_t w[48];
            uint8_t q[48], e[2];
            if (oracle_mx8_quantize(w, 1, 48, q, e) != -1) return 5;   /* K % 32 != 0 */
        }
    }
    printf("sanitized oracle run ok\n");
    return 0;
}
