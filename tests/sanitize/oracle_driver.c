/* Test support: exercises every entry point of the CPU oracle on small
 * seeded inputs (both formats, every norm, N:M patterns with M up to 16,
 * ragged K, a row subset, the SiLU source, weights with a row stride,
 * dequantization), built with the host address and undefined-behaviour
 * sanitizers; prints "ok" when every call succeeds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_prepare(const void *x, int xdt, int64_t T, int64_t K, int64_t ldx, int norm, const void *gamma,
               const void *beta, int gdt, float eps, int N, int M, int fmt, const int64_t *rows, int64_t nrows,
               uint8_t *mask, uint8_t *b_codes, uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales,
               float *gscale, float *xhat_out, float *deqb_out, float *resid_out);
int or_prepare_swiglu(const float *gu, int64_t T, int64_t K, int64_t ld, int N, int M, int fmt, const int64_t *rows,
                      int64_t nrows, uint8_t *mask, uint8_t *b_codes, uint8_t *b_scales, uint8_t *r_codes,
                      uint8_t *r_scales, float *gscale, float *xhat_out, float *deqb_out, float *resid_out);
int or_quantize_weight(const void *w, int wdt, int64_t E, int64_t Nout, int64_t K, int64_t ldw, int fmt,
                       uint8_t *codes, uint8_t *scales, float *gscale);
int or_quantize_rows(const void *w, int wdt, int64_t nrows, int64_t K, int fmt, float G, uint8_t *codes,
                     uint8_t *scales);
int or_dequant(const uint8_t *codes, const uint8_t *scales, int64_t nrows, int64_t K, int fmt, float G,
               double *out);
int or_normalize(const void *x, int xdt, int64_t T, int64_t K, int64_t ldx, int norm, const void *gamma,
                 const void *beta, int gdt, float eps, float *xhat);
void or_select_group(const float *v, int M, int N, uint8_t *keep);
float or_exp32(float y);
float or_silu32(float g);

static uint64_t state = 12345;
static float uniform(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((state >> 40) & 0xFFFFFF) / 16777216.0f;
}
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFF + ((u >> 16) & 1);
    return (uint16_t)(u >> 16);
}

int main(void) {
    int fails = 0;
    const int64_t T = 5, Ks[2] = {256, 320};
    for (int ki = 0; ki < 2; ki++) {
        const int64_t K = Ks[ki], ld = K + 8;
        uint16_t *x = malloc(sizeof(uint16_t) * T * ld), *g = malloc(sizeof(uint16_t) * K),
                 *b = malloc(sizeof(uint16_t) * K);
        for (int64_t i = 0; i < T * ld; i++) x[i] = bf16_of((uniform() - 0.5f) * (i % 37 == 0 ? 80.0f : 2.0f));
        for (int64_t i = 0; i < K; i++) {
            g[i] = bf16_of(1.0f + 0.1f * (uniform() - 0.5f));
            b[i] = bf16_of(0.1f * (uniform() - 0.5f));
        }
        const int nm[6][2] = {{2, 4}, {1, 2}, {4, 8}, {8, 16}, {0, 4}, {1, 1}};
        for (int fmt = 0; fmt < 2; fmt++) {
            const int B = fmt == 0 ? 32 : 16;
            if (K % B) continue;
            for (int norm = 0; norm < 3; norm++) {
                for (int p = 0; p < 6; p++) {
                    const int64_t rows[2] = {4, 1};
                    for (int sub = 0; sub < 2; sub++) {
                        const int64_t nr = sub ? 2 : T;
                        uint8_t *mask = malloc(nr * K / 8), *bc = malloc(nr * K / 2), *bs = malloc(nr * K / B),
                                *rc = malloc(nr * K / 2), *rs = malloc(nr * K / B);
                        float gs, *xh = malloc(sizeof(float) * nr * K), *dq = malloc(sizeof(float) * nr * K),
                                  *re = malloc(sizeof(float) * nr * K);
                        if (or_prepare(x, 1, T, K, ld, norm, g, b, 1, 1e-5f, nm[p][0], nm[p][1], fmt,
                                       sub ? rows : NULL, nr, mask, bc, bs, rc, rs, &gs, xh, dq, re) != 0)
                            fails++;
                        double *out = malloc(sizeof(double) * nr * K);
                        if (or_dequant(bc, bs, nr, K, fmt, gs, out) != 0) fails++;
                        free(out);
                        free(mask); free(bc); free(bs); free(rc); free(rs); free(xh); free(dq); free(re);
                    }
                }
            }
            /* SiLU source and weights with a row stride */
            float *gu = malloc(sizeof(float) * T * (2 * K + 4));
            for (int64_t i = 0; i < T * (2 * K + 4); i++) gu[i] = 6.0f * (uniform() - 0.5f);
            uint8_t *mask = malloc(T * K / 8), *bc = malloc(T * K / 2), *bs = malloc(T * K / B),
                    *rc = malloc(T * K / 2), *rs = malloc(T * K / B);
            float gs;
            if (or_prepare_swiglu(gu, T, K, 2 * K + 4, 2, 4, fmt, NULL, T, mask, bc, bs, rc, rs, &gs, NULL, NULL,
                                  NULL) != 0)
                fails++;
            uint8_t *wc = malloc(2 * 3 * K / 2), *wsc = malloc(2 * 3 * K / B);
            float wg[2];
            if (or_quantize_weight(x, 1, 2, 2, K, ld, fmt, wc, wsc, wg) != 0) fails++;
            if (or_quantize_rows(x, 1, 3, K, fmt, 1.0f, wc, wsc) != 0) fails++;
            float *xh = malloc(sizeof(float) * T * K);
            if (or_normalize(x, 1, T, K, ld, 2, g, b, 1, 1e-5f, xh) != 0) fails++;
            free(xh); free(gu); free(mask); free(bc); free(bs); free(rc); free(rs); free(wc); free(wsc);
        }
        free(x); free(g); free(b);
    }
    float v[16];
    uint8_t keep[16];
    for (int i = 0; i < 16; i++) v[i] = uniform() - 0.5f;
    or_select_group(v, 16, 5, keep);
    for (float y = -100.0f; y < 100.0f; y += 0.37f) {
        if (!(or_exp32(y) >= 0.0f)) fails++;
        (void)or_silu32(y);
    }
    if (fails == 0) printf("ok\n");
    else printf("%d failures\n", fails);
    return fails == 0 ? 0 : 1;
}
