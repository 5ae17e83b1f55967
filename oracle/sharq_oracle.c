/*
 * Plain CPU oracle for the SharQ hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * What it computes (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract): for every
 * activation tensor, normalize it, choose an N:M mask from its own
 * magnitudes so that the large (outlier) elements form a sparse backbone,
 * quantize that backbone to FP4 with block scales, subtract the
 * dequantized backbone from the normalized tensor to get the dense residual,
 * and quantize the residual to FP4 too; the layer output is
 * backbone.W + residual.W with one FP4 weight payload.  The pages give no
 * formulas, so every step below takes the plainest reading:
 *
 *   norm      RMSNorm: ss = serial FP64 sum of x^2, r = (float)(1/sqrt(ss/K+eps))
 *             evaluated in double, xhat = fl32(fl32(x*r)*gamma).
 *             LayerNorm: FP64 two-pass mean and variance, mu and r rounded
 *             to float, xhat = fl32(fl32(fl32(fl32(x-mu)*r)*gamma)+beta).
 *             None: xhat = x.
 *   mask      per group of M consecutive elements along K, keep the N largest
 *             |xhat| (compared as the IEEE bit pattern without sign); equal
 *             magnitudes go to the lower index.
 *   MXFP4     32-element blocks, E8M0 scale 2^E with E = floor(log2 amax) - 2
 *             (the OCP MX shared-exponent rule for E2M1), clamped to
 *             [-127, 127], amax = 0 giving E = -127; element codes are the
 *             E2M1 value nearest to v*2^-E, ties to the even code, saturating
 *             at 6, and a zero magnitude is always the code 0x0.
 *   NVFP4     16-element blocks with an E4M3 scale and one FP32 scale G per
 *             tensor: G = fl32(amax(tensor)/2688) (1 if that is not > 0),
 *             s = E4M3(fl32(amax(block)/fl32(6G))) rounded to nearest even
 *             and saturated at 448, D = fl32(s*G), code = E2M1(fl32(v/D)),
 *             dequantized value fl32(grid[code]*D).  The backbone and the
 *             residual of one tensor share G.
 *   residual  R = fl32(xhat - deq(Q(S))).
 *
 * Build: plain C99, -O2 -ffp-contract=off, no fast-math; x86-64 SSE floats
 * so every float operation is rounded to single precision on its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_DT_F16 = 0, OR_DT_BF16 = 1, OR_DT_F32 = 2 };
enum { OR_NORM_NONE = 0, OR_NORM_RMS = 1, OR_NORM_LAYER = 2 };
enum { OR_FMT_MXFP4 = 0, OR_FMT_NVFP4 = 1 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENOMEM = 2 };

/* ------------------------------------------------------------------ */
/* element types                                                       */
/* ------------------------------------------------------------------ */

static float float_from_bits(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t bits_from_float(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

/* bfloat16 is the top half of a float32. */
static float decode_bf16(uint16_t h) { return float_from_bits((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static float decode_f16(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

static float load_elem(const void *p, int dt, int64_t i)
{
    if (dt == OR_DT_BF16) return decode_bf16(((const uint16_t *)p)[i]);
    if (dt == OR_DT_F16) return decode_f16(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

/* E2M1 magnitudes, indexed by the 3-bit magnitude code. */
static const float E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Nearest E2M1 magnitude code of a >= 0, ties to the even code, saturating.
 * The decision points are the midpoints between neighbouring grid values. */
static int e2m1_magnitude_code(float a)
{
    if (a <= 0.25f) return 0; /* midpoint 0.25: tie -> code 0 */
    if (a < 0.75f) return 1;  /* midpoint 0.75: tie -> code 2 */
    if (a <= 1.25f) return 2; /* midpoint 1.25: tie -> code 2 */
    if (a < 1.75f) return 3;  /* midpoint 1.75: tie -> code 4 */
    if (a <= 2.5f) return 4;  /* midpoint 2.5:  tie -> code 4 */
    if (a < 3.5f) return 5;   /* midpoint 3.5:  tie -> code 6 */
    if (a <= 5.0f) return 6;  /* midpoint 5:    tie -> code 6 */
    return 7;                 /* 6 and above saturate */
}

/* Sign-magnitude E2M1 code of u; zero magnitude is always the code 0x0. */
uint8_t or_e2m1_encode(float u)
{
    int c = e2m1_magnitude_code(fabsf(u));
    if (c == 0) return 0;
    return (uint8_t)((signbit(u) ? 8 : 0) | c);
}

float or_e2m1_decode(uint8_t code)
{
    float v = E2M1_GRID[code & 7];
    return (code & 8) ? -v : v;
}

void or_e2m1_encode_n(const float *u, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = or_e2m1_encode(u[i]);
}

/* OCP MX shared exponent for E2M1 elements (largest element exponent 2). */
int or_mx_exponent(float amax)
{
    if (amax == 0.0f) return -127;
    int e = ilogbf(amax) - 2; /* ilogbf is exact for subnormals too */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

void or_mx_exponent_n(const float *amax, int64_t n, int16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (int16_t)or_mx_exponent(amax[i]);
}

/* E4M3 (no infinities, 0x7F/0xFF are NaN): bias 7, largest finite 448. */
uint8_t or_e4m3_encode(float x);

void or_e4m3_encode_n(const float *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = or_e4m3_encode(x[i]);
}

float or_e4m3_decode(uint8_t b)
{
    int e = (b >> 3) & 15, m = b & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)((b & 0x80) ? -v : v);
}

/* Round a non-negative float to E4M3, nearest with ties to even, saturating
 * at the largest finite value 448 (no NaN is ever produced). */
uint8_t or_e4m3_encode(float x)
{
    if (!(x > 0.0f)) return 0;
    if (x >= 448.0f) return 0x7E;
    int e = ilogbf(x);
    if (e < -6) e = -6;                         /* subnormal quantum is 2^-9 */
    double q = ldexp(1.0, e - 3);               /* 3 fraction bits */
    double n = nearbyint((double)x / q);        /* exact scaling, then RNE */
    double v = n * q;
    if (v > 448.0) v = 448.0;
    if (v == 0.0) return 0;
    int ev = ilogb(v);
    if (ev < -6) return (uint8_t)(int)(v / ldexp(1.0, -9)); /* subnormal */
    int frac = (int)(v / ldexp(1.0, ev) * 8.0) - 8;
    return (uint8_t)(((ev + 7) << 3) | frac);
}

/* ------------------------------------------------------------------ */
/* normalization, mask                                                 */
/* ------------------------------------------------------------------ */

static void normalize_row(const float *x, int64_t K, int norm, const float *g,
                          const float *b, float eps, float *out)
{
    if (norm == OR_NORM_NONE) {
        for (int64_t k = 0; k < K; k++) out[k] = x[k];
        return;
    }
    if (norm == OR_NORM_RMS) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) ss += (double)x[k] * (double)x[k];
        float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        for (int64_t k = 0; k < K; k++) {
            float t = x[k] * r;
            out[k] = t * g[k];
        }
        return;
    }
    /* LayerNorm */
    double s = 0.0;
    for (int64_t k = 0; k < K; k++) s += (double)x[k];
    double mud = s / (double)K;
    double v = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double d = (double)x[k] - mud;
        v += d * d;
    }
    double vd = v / (double)K;
    float mu = (float)mud;
    float r = (float)(1.0 / sqrt(vd + (double)eps));
    for (int64_t k = 0; k < K; k++) {
        float t = x[k] - mu;
        t = t * r;
        t = t * g[k];
        out[k] = t + (b ? b[k] : 0.0f);
    }
}

/* Keep the N largest magnitudes of one group of M values; equal magnitudes
 * rank the lower index first.  keep[i] is set to 1 or 0. */
void or_select_group(const float *v, int M, int N, uint8_t *keep)
{
    for (int k = 0; k < M; k++) {
        uint32_t key_k = bits_from_float(v[k]) & 0x7FFFFFFFu;
        int rank = 0;
        for (int i = 0; i < M; i++) {
            if (i == k) continue;
            uint32_t key_i = bits_from_float(v[i]) & 0x7FFFFFFFu;
            if (key_i > key_k || (key_i == key_k && i < k)) rank++;
        }
        keep[k] = rank < N;
    }
}

/* ------------------------------------------------------------------ */
/* block quantizers                                                    */
/* ------------------------------------------------------------------ */

/* MXFP4 block of 32: codes[i] unpacked, returns the scale byte, deq[i] set. */
static uint8_t mx_block(const float *v, uint8_t *codes, float *deq)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    int E = or_mx_exponent(amax);
    for (int i = 0; i < 32; i++) {
        float u = ldexpf(v[i], -E);
        uint8_t c = or_e2m1_encode(u);
        codes[i] = c;
        deq[i] = ldexpf(or_e2m1_decode(c), E);
    }
    return (uint8_t)(E + 127);
}

/* NVFP4 block of 16 with tensor scale G (G6 = fl32(6*G)). */
static uint8_t nv_block(const float *v, float G, uint8_t *codes, float *deq)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float G6 = 6.0f * G;
    float t = amax / G6;
    uint8_t s = or_e4m3_encode(t);
    float D = or_e4m3_decode(s) * G;
    for (int i = 0; i < 16; i++) {
        if (s == 0) {
            codes[i] = 0;
            deq[i] = 0.0f;
            continue;
        }
        float u = v[i] / D;
        uint8_t c = or_e2m1_encode(u);
        codes[i] = c;
        float mag = E2M1_GRID[c & 7] * D;
        deq[i] = (c & 8) ? -mag : mag;
    }
    return s;
}

float or_nv_global_scale(float amax)
{
    float G = amax / 2688.0f;
    if (!(G > 0.0f)) G = 1.0f;
    return G;
}

/* Quantize one row of K values; codes packed two per byte, even k in the low
 * nibble; one scale byte per block; deq (nullable) receives dequantized values. */
static void quantize_row(const float *v, int64_t K, int fmt, float G, uint8_t *codes_packed,
                         uint8_t *scales, float *deq)
{
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    uint8_t c[32];
    float d[32];
    for (int64_t b0 = 0; b0 < K; b0 += B) {
        uint8_t sc = fmt == OR_FMT_MXFP4 ? mx_block(v + b0, c, d) : nv_block(v + b0, G, c, d);
        scales[b0 / B] = sc;
        for (int i = 0; i < B; i += 2)
            codes_packed[(b0 + i) / 2] = (uint8_t)(c[i] | (c[i + 1] << 4));
        if (deq)
            for (int i = 0; i < B; i++) deq[b0 + i] = d[i];
    }
}

static int check_shape(int64_t K, int N, int M, int fmt)
{
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    if (fmt != OR_FMT_MXFP4 && fmt != OR_FMT_NVFP4) return OR_EINVAL;
    if (M < 1 || N < 0 || N > M || K <= 0 || K % B || K % M) return OR_EINVAL;
    return OR_OK;
}

/* One prepared row i from its normalized values xh[K]: mask, backbone
 * S = mask ? xh : +0 quantized, residual R = xh - deq(Q(S)) quantized
 * (scratch S, dq, R, keep are K long; traces nullable). */
static void decompose_row(const float *xh, int64_t K, int N, int M, int fmt, float G, int64_t i,
                          float *S, float *dq, float *R, uint8_t *keep, uint8_t *mask,
                          uint8_t *b_codes, uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales,
                          float *xhat_out, float *deqb_out, float *resid_out)
{
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    /* mask and backbone */
    for (int64_t g0 = 0; g0 < K; g0 += M) or_select_group(xh + g0, M, N, keep + g0);
    for (int64_t k = 0; k < K; k++) S[k] = keep[k] ? xh[k] : 0.0f;
    if (mask) {
        uint8_t *mrow = mask + i * (K / 8);
        for (int64_t j = 0; j < K / 8; j++) mrow[j] = 0;
        for (int64_t k = 0; k < K; k++)
            if (keep[k]) mrow[k / 8] |= (uint8_t)(1u << (k % 8));
    }
    quantize_row(S, K, fmt, G, b_codes + i * (K / 2), b_scales + i * (K / B), dq);
    /* residual against the dequantized backbone */
    for (int64_t k = 0; k < K; k++) R[k] = xh[k] - dq[k];
    if (xhat_out) memcpy(xhat_out + i * K, xh, sizeof(float) * K);
    if (deqb_out) memcpy(deqb_out + i * K, dq, sizeof(float) * K);
    if (resid_out) memcpy(resid_out + i * K, R, sizeof(float) * K);
    quantize_row(R, K, fmt, G, r_codes + i * (K / 2), r_scales + i * (K / B), NULL);
}

/* ------------------------------------------------------------------ */
/* SiLU(gate) * up (the activation feeding a down projection)          */
/* ------------------------------------------------------------------ */

/* e^y in float, as a fixed sequence of correctly rounded float operations
 * (so any IEEE implementation of the same steps gives the same bits):
 * Cody-Waite reduction y = n ln2 + r with n = rint(y log2 e) and ln2 split
 * into a 15-bit head and a tail, e^r by its degree-6 Taylor polynomial in
 * Horner form with each step one fused multiply-add (one rounding), then
 * scaling by 2^n.  Defined as 0 below -87 (so results are never subnormal)
 * and +inf above 88.  About 2 ulp from the true e^y. */
float or_exp32(float y)
{
    if (!(y <= 88.0f)) return INFINITY;
    if (y < -87.0f) return 0.0f;
    float n = nearbyintf(y * 1.44269504f);
    float r = (y - n * 0.693145752f) - n * 1.42860677e-6f;
    float p = 0.00138888889f;              /* 1/720 */
    p = fmaf(p, r, 0.00833333333f);        /* 1/120 */
    p = fmaf(p, r, 0.0416666667f);         /* 1/24 */
    p = fmaf(p, r, 0.166666667f);          /* 1/6 */
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* SiLU(g) = g / (1 + e^-g), each step rounded to float. */
float or_silu32(float g)
{
    float d = 1.0f + or_exp32(-g);
    return g / d;
}

void or_silu32_n(const float *g, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = or_silu32(g[i]);
}

/* ------------------------------------------------------------------ */
/* public entry points                                                 */
/* ------------------------------------------------------------------ */

/* Normalized rows only (used for tie analysis and for error reports). */
int or_normalize(const void *x, int xdt, int64_t T, int64_t K, int64_t ldx, int norm,
                 const void *gamma, const void *beta, int gdt, float eps, float *xhat)
{
    float *row = malloc(sizeof(float) * K), *g = malloc(sizeof(float) * K),
          *b = malloc(sizeof(float) * K);
    if (!row || !g || !b) { free(row); free(g); free(b); return OR_ENOMEM; }
    for (int64_t k = 0; k < K; k++) {
        g[k] = gamma ? load_elem(gamma, gdt, k) : 1.0f;
        b[k] = beta ? load_elem(beta, gdt, k) : 0.0f;
    }
    for (int64_t t = 0; t < T; t++) {
        for (int64_t k = 0; k < K; k++) row[k] = load_elem(x, xdt, t * ldx + k);
        normalize_row(row, K, norm, g, beta ? b : NULL, eps, xhat + t * K);
    }
    free(row); free(g); free(b);
    return OR_OK;
}

/*
 * Prepare one activation tensor X[T][K] (row stride ldx elements).
 * rows/nrows select which rows are produced (rows == NULL: all T rows, in
 * order); the NVFP4 tensor scale is always taken over all T rows.
 * Outputs, per produced row i:
 *   mask     [i][K/8]  bit k%8 of byte k/8 set if element k is kept
 *   b_codes  [i][K/2], b_scales [i][K/B]   backbone
 *   r_codes  [i][K/2], r_scales [i][K/B]   residual
 *   gscale   one float (NVFP4 tensor scale; 1.0 for MXFP4)
 * Optional float traces [i][K] (nullable): normalized values, dequantized
 * backbone, residual before its quantization.
 */
int or_prepare(const void *x, int xdt, int64_t T, int64_t K, int64_t ldx, int norm,
               const void *gamma, const void *beta, int gdt, float eps, int N, int M, int fmt,
               const int64_t *rows, int64_t nrows, uint8_t *mask, uint8_t *b_codes,
               uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales, float *gscale,
               float *xhat_out, float *deqb_out, float *resid_out)
{
    if (check_shape(K, N, M, fmt) != OR_OK || T < 0 || ldx < K) return OR_EINVAL;
    float *row = malloc(sizeof(float) * K), *xh = malloc(sizeof(float) * K),
          *g = malloc(sizeof(float) * K), *bt = malloc(sizeof(float) * K),
          *S = malloc(sizeof(float) * K), *dq = malloc(sizeof(float) * K),
          *R = malloc(sizeof(float) * K);
    uint8_t *keep = malloc(K);
    int rc = OR_OK;
    if (!row || !xh || !g || !bt || !S || !dq || !R || !keep) { rc = OR_ENOMEM; goto out; }
    for (int64_t k = 0; k < K; k++) {
        g[k] = gamma ? load_elem(gamma, gdt, k) : 1.0f;
        bt[k] = beta ? load_elem(beta, gdt, k) : 0.0f;
    }

    float G = 1.0f;
    if (fmt == OR_FMT_NVFP4) {
        float amax = 0.0f;
        for (int64_t t = 0; t < T; t++) {
            for (int64_t k = 0; k < K; k++) row[k] = load_elem(x, xdt, t * ldx + k);
            normalize_row(row, K, norm, g, beta ? bt : NULL, eps, xh);
            for (int64_t k = 0; k < K; k++)
                if (fabsf(xh[k]) > amax) amax = fabsf(xh[k]);
        }
        G = or_nv_global_scale(amax);
    }
    if (gscale) *gscale = G;

    int64_t nr = rows ? nrows : T;
    for (int64_t i = 0; i < nr; i++) {
        int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) { rc = OR_EINVAL; goto out; }
        for (int64_t k = 0; k < K; k++) row[k] = load_elem(x, xdt, t * ldx + k);
        normalize_row(row, K, norm, g, beta ? bt : NULL, eps, xh);
        decompose_row(xh, K, N, M, fmt, G, i, S, dq, R, keep, mask, b_codes, b_scales, r_codes,
                      r_scales, xhat_out, deqb_out, resid_out);
    }
out:
    free(row); free(xh); free(g); free(bt); free(S); free(dq); free(R); free(keep);
    return rc;
}

/*
 * Quantize W[E][Nout][K] (row stride ldw elements, expert stride Nout*ldw)
 * into one FP4 payload: codes [E][Nout][K/2], scales [E][Nout][K/B],
 * gscale[E] (NVFP4 per-expert tensor scale; 1.0 for MXFP4).
 */
int or_quantize_weight(const void *w, int wdt, int64_t E, int64_t Nout, int64_t K, int64_t ldw,
                       int fmt, uint8_t *codes, uint8_t *scales, float *gscale)
{
    if (check_shape(K, 1, 1, fmt) != OR_OK || E < 1 || Nout < 0 || ldw < K) return OR_EINVAL;
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    float *row = malloc(sizeof(float) * K);
    if (!row) return OR_ENOMEM;
    for (int64_t e = 0; e < E; e++) {
        float G = 1.0f;
        if (fmt == OR_FMT_NVFP4) {
            float amax = 0.0f;
            for (int64_t n = 0; n < Nout; n++)
                for (int64_t k = 0; k < K; k++) {
                    float a = fabsf(load_elem(w, wdt, (e * Nout + n) * ldw + k));
                    if (a > amax) amax = a;
                }
            G = or_nv_global_scale(amax);
        }
        if (gscale) gscale[e] = G;
        for (int64_t n = 0; n < Nout; n++) {
            for (int64_t k = 0; k < K; k++) row[k] = load_elem(w, wdt, (e * Nout + n) * ldw + k);
            quantize_row(row, K, fmt, G, codes + (e * Nout + n) * (K / 2),
                         scales + (e * Nout + n) * (K / B), NULL);
        }
    }
    free(row);
    return OR_OK;
}

/* Quantize rows W[nrows][K] (row stride K) with a given tensor scale G
 * (NVFP4; ignored for MXFP4) -- used to check a sample of a large weight. */
int or_quantize_rows(const void *w, int wdt, int64_t nrows, int64_t K, int fmt, float G,
                     uint8_t *codes, uint8_t *scales)
{
    if (check_shape(K, 1, 1, fmt) != OR_OK || nrows < 0) return OR_EINVAL;
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    float *row = malloc(sizeof(float) * K);
    if (!row) return OR_ENOMEM;
    for (int64_t n = 0; n < nrows; n++) {
        for (int64_t k = 0; k < K; k++) row[k] = load_elem(w, wdt, n * K + k);
        quantize_row(row, K, fmt, G, codes + n * (K / 2), scales + n * (K / B), NULL);
    }
    free(row);
    return OR_OK;
}

/* Exact FP64 values of FP4 rows: codes [rows][K/2], scales [rows][K/B]. */
int or_dequant(const uint8_t *codes, const uint8_t *scales, int64_t nrows, int64_t K, int fmt,
               float G, double *out)
{
    if (check_shape(K, 1, 1, fmt) != OR_OK) return OR_EINVAL;
    int B = fmt == OR_FMT_MXFP4 ? 32 : 16;
    for (int64_t r = 0; r < nrows; r++)
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte = codes[r * (K / 2) + k / 2];
            uint8_t c = (k % 2) ? (byte >> 4) : (byte & 15);
            uint8_t s = scales[r * (K / B) + k / B];
            double v = (double)or_e2m1_decode(c);
            if (fmt == OR_FMT_MXFP4)
                v = ldexp(v, (int)s - 127);
            else
                v = v * (double)or_e4m3_decode(s) * (double)G;
            out[r * K + k] = v;
        }
    return OR_OK;
}

/*
 * Prepare the input of a down projection straight from the gate/up product:
 * row t of GU (row stride ld floats) holds the gate in columns [0, K) and
 * the up projection in [K, 2K); the activation is
 *   xhat[k] = fl32(SiLU(gate[k]) * up[k])   (no normalization)
 * and the rest is exactly or_prepare's (mask, backbone, residual, NVFP4
 * tensor scale over all T rows).  Same outputs and traces as or_prepare.
 */
int or_prepare_swiglu(const float *gu, int64_t T, int64_t K, int64_t ld, int N, int M, int fmt,
                      const int64_t *rows, int64_t nrows, uint8_t *mask, uint8_t *b_codes,
                      uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales, float *gscale,
                      float *xhat_out, float *deqb_out, float *resid_out)
{
    if (check_shape(K, N, M, fmt) != OR_OK || T < 0 || ld < 2 * K) return OR_EINVAL;
    float *xh = malloc(sizeof(float) * K), *S = malloc(sizeof(float) * K),
          *dq = malloc(sizeof(float) * K), *R = malloc(sizeof(float) * K);
    uint8_t *keep = malloc(K);
    int rc = OR_OK;
    if (!xh || !S || !dq || !R || !keep) { rc = OR_ENOMEM; goto out; }
    float G = 1.0f;
    if (fmt == OR_FMT_NVFP4) {
        float amax = 0.0f;
        for (int64_t t = 0; t < T; t++)
            for (int64_t k = 0; k < K; k++) {
                float v = or_silu32(gu[t * ld + k]) * gu[t * ld + K + k];
                if (fabsf(v) > amax) amax = fabsf(v);
            }
        G = or_nv_global_scale(amax);
    }
    if (gscale) *gscale = G;
    int64_t nr = rows ? nrows : T;
    for (int64_t i = 0; i < nr; i++) {
        int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) { rc = OR_EINVAL; goto out; }
        for (int64_t k = 0; k < K; k++) xh[k] = or_silu32(gu[t * ld + k]) * gu[t * ld + K + k];
        decompose_row(xh, K, N, M, fmt, G, i, S, dq, R, keep, mask, b_codes, b_scales, r_codes,
                      r_scales, xhat_out, deqb_out, resid_out);
    }
out:
    free(xh); free(S); free(dq); free(R); free(keep);
    return rc;
}
