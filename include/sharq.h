/*
 * sharq.h -- C ABI of the SharQ hot path on AMD Instinct MI355X (gfx950).
 *
 * Method (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract; arXiv 2606.26587): each activation tensor of a linear
 * layer is cut into two FP4 parts.  An N:M mask chosen from the tensor's own
 * values keeps the large-magnitude elements (where the outliers live); those
 * form a sparse backbone that is quantized to FP4.  What the quantized
 * backbone fails to represent -- the masked-out elements plus the backbone's
 * own rounding error -- is a dense residual, also quantized to FP4.  The
 * layer output adds the backbone product and the residual product, both
 * against one FP4 copy of the weight.  Normalization, masking and residual
 * formation run as one fused operator.
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device (or managed) memory; the library never
 *     allocates or frees memory.  Scratch space comes from the caller as a
 *     workspace argument sized by the *_workspace_size() helpers.
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = the default
 *     stream) and runs asynchronously; no call synchronizes with the host.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns its status code and enqueues nothing.  SHARQ_ERR_HIP reports a
 *     failed launch (sharq_last_hip_error() gives the hipError_t); faults
 *     inside a kernel surface at the caller's next synchronization, as usual
 *     with HIP.  On any error the outputs are unspecified.
 *   - Check mode: with the environment variable SHARQ_DEBUG=1 every entry
 *     point also waits for its own launches on `stream` (except while the
 *     stream is being captured into a HIP graph) and returns SHARQ_ERR_HIP,
 *     with the entry point's name and the HIP error on stderr, when they
 *     failed.  The variable is read on every call.
 *   - Element formats:
 *       E2M1   FP4 code: bit 3 sign, bits 0-2 magnitude index into
 *              {0, 0.5, 1, 1.5, 2, 3, 4, 6}; a zero magnitude is always 0x0.
 *              Two codes per byte, element k in the low nibble when k is even.
 *       MXFP4  E2M1 + one E8M0 scale byte per 32 elements along K:
 *              scale 2^(byte-127), exponent floor(log2 amax) - 2 (OCP MX v1.0).
 *       NVFP4  E2M1 + one E4M3 scale byte per 16 elements along K, times one
 *              FP32 scale per tensor, amax(tensor)/2688.
 *       NVFP4_SP24  NVFP4 whose backbone is stored in the compressed form of
 *              gfx950's 2:4 sparse f16 matrix instruction, so that products
 *              run the backbone on it (2:4 masks only, K % 128 == 0,
 *              T*K/2 < 2^32).  Per row and K tile (elements e = 0..127 of
 *              the tile) the backbone takes 48 bytes: bytes 4c..4c+3 hold
 *              chunk c = 4p + 2h + u (p, h, u in {0, 1}): the kept codes of
 *              elements 32p + 16u + 8h + [0, 8), then of
 *              64 + 32p + 16u + 8h + [0, 8), two per group of four in
 *              ascending position, code v of the chunk in nibble v % 2 of
 *              byte v / 2; bytes 32 + 4(2p + h) .. +3 hold in bits
 *              16u + 2v, 16u + 2v + 1 the position (0..3) within its group
 *              of code v of chunk 4p + 2h + u.  These 48-byte rows are
 *              K-tiled like the other arrays (T*K*3/8 bytes).  The tile's
 *              eight backbone block scales are stored in the order of blocks
 *              0, 1, 4, 5, 2, 3, 6, 7 (block b = elements 16b..16b+15).  The
 *              residual, the mask and the tensor scale are those of NVFP4;
 *              weights are NVFP4 (sharq_quantize_weight treats NVFP4_SP24 as
 *              NVFP4).
 *   - The N:M mask keeps, in every group of M consecutive elements along K,
 *     the N elements of largest magnitude; equal magnitudes favour the lower
 *     index.  Mask bitmap: bit k%8 of byte k/8 of the row.
 *   - K-tiled layout of every FP4 code and scale array ("rows" = T for
 *     prepared activations, nout for one expert's weights): K is cut into
 *     tiles of 128 elements, the last one w = K - 128*floor(K/128) wide when
 *     K is not a multiple of 128.  Tile t is stored after tiles 0..t-1 and
 *     holds all rows back to back, each row with the tile's codes (w/2 bytes,
 *     element k in the low nibble when k is even) or scales (w/B bytes):
 *       byte of element k of row r = floor(k/128)*rows*(128/P)
 *                                    + r*(w_t/P) + (k mod 128)/P,
 *     P = 2 for codes, P = B (32 MX, 16 NV) for scales, w_t the width of
 *     k's tile.  Total size rows*K/P, the same as row-major.  One K step of
 *     the products then reads one contiguous run per array.
 */
#ifndef SHARQ_H
#define SHARQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHARQ_ABI_VERSION 7

#if defined(__GNUC__)
#define SHARQ_API __attribute__((visibility("default")))
#else
#define SHARQ_API
#endif

typedef enum {
    SHARQ_OK = 0,
    SHARQ_ERR_NULL = 1,        /* a required pointer is NULL                    */
    SHARQ_ERR_SHAPE = 2,       /* a size is negative, K not a multiple of the   */
                               /* block (32 MX / 16 NV) or of 128 for products, */
                               /* or a leading dimension is too small           */
    SHARQ_ERR_NM = 3,          /* not 0 <= N <= M, or M not in {1,2,4,8,16}, or */
                               /* M does not divide K                           */
    SHARQ_ERR_DTYPE = 4,       /* unsupported element type                      */
    SHARQ_ERR_ALIGN = 5,       /* pointer or row stride less aligned than its   */
                               /* argument requires                             */
    SHARQ_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required       */
    SHARQ_ERR_UNSUPPORTED = 7, /* format / norm / combination not built         */
    SHARQ_ERR_HIP = 8          /* a HIP call or kernel launch failed            */
} sharq_status;

typedef enum { SHARQ_F16 = 0, SHARQ_BF16 = 1, SHARQ_F32 = 2 } sharq_dtype;
typedef enum { SHARQ_NORM_NONE = 0, SHARQ_NORM_RMS = 1, SHARQ_NORM_LAYER = 2 } sharq_norm;
typedef enum { SHARQ_MXFP4 = 0, SHARQ_NVFP4 = 1, SHARQ_NVFP4_SP24 = 2 } sharq_format;

/* Version of this ABI (SHARQ_ABI_VERSION). */
SHARQ_API int sharq_abi_version(void);

/* Static, NUL-terminated description of a status code. */
SHARQ_API const char *sharq_status_string(int status);

/* The hipError_t (0 = hipSuccess) of the calling thread's most recent entry
 * point call that reached HIP (launches, and in check mode the wait); calls
 * rejected by argument validation leave it unchanged. */
SHARQ_API int sharq_last_hip_error(void);

/* Bytes of workspace sharq_prepare needs for T rows (0 for MXFP4). */
SHARQ_API size_t sharq_prepare_workspace_size(int64_t T, int64_t K, int32_t fmt);

/*
 * sharq_prepare -- the fused preparation operator (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract:
 * normalization, mask generation and residual construction in one
 * operator; backbone and residual as in the decomposition it describes).
 *
 * Per row t of X (T rows, K columns, row stride ldx elements):
 *   xhat = norm(x)           NONE: x;  RMS: x * r * gamma with
 *                            r = fl32(1/sqrt(sum(x^2)/K + eps)) (sum in FP64);
 *                            LAYER: ((x - mu) * r) * gamma + beta
 *   mask = top-N |xhat| of every M-group along K
 *   S    = mask ? xhat : 0;             backbone = Q(S)
 *   R    = xhat - deq(backbone);        residual = Q(R)
 * where Q is MXFP4 or NVFP4 (the NVFP4 tensor scale G = amax(xhat)/2688 is
 * shared by backbone and residual and written to *global_scale).
 *
 *   x            [T][ldx] F16 or BF16, 16-byte aligned, ldx*2 % 16 == 0
 *   gamma, beta  [K] same type as x; gamma required for RMS and LAYER, beta
 *                optional for LAYER (NULL = 0), both ignored for NONE
 *   eps          added to the mean square / variance
 *   n, m         N:M mask, 0 <= n <= m, m in {1,2,4,8,16}, K % m == 0
 *   fmt          SHARQ_MXFP4 (K % 32 == 0), SHARQ_NVFP4 (K % 16 == 0) or
 *                SHARQ_NVFP4_SP24 (n = 2, m = 4, K % 128 == 0, T*K/2 < 2^32;
 *                SHARQ_ERR_NM / SHARQ_ERR_SHAPE otherwise)
 *   mask         [T][K/8] row-major bitmap or NULL (not written)
 *   b_codes      T*K/2 bytes, backbone E2M1 codes, K-tiled, 4-byte aligned
 *                (NVFP4_SP24: T*K*3/8 bytes in the compressed form)
 *   b_scales     T*K/B bytes, backbone block scales (E8M0 or E4M3), K-tiled
 *                (NVFP4_SP24: in its block order)
 *   r_codes      T*K/2 bytes, residual codes, K-tiled, 4-byte aligned
 *   r_scales     T*K/B bytes, residual block scales, K-tiled
 *   global_scale one device float: NVFP4 tensor scale (written); MXFP4: may
 *                be NULL, otherwise 1.0f is written
 *   workspace    sharq_prepare_workspace_size() bytes (NVFP4 only)
 * All outputs are dense arrays owned by the caller.  T == 0 is a valid
 * no-op; T must stay below 2^31 - 64 (SHARQ_ERR_SHAPE otherwise).
 */
SHARQ_API sharq_status sharq_prepare(const void *x, int32_t x_dtype, int64_t T, int64_t K, int64_t ldx,
                           int32_t norm, const void *gamma, const void *beta, float eps,
                           int32_t n, int32_t m, int32_t fmt, uint8_t *mask, uint8_t *b_codes,
                           uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales,
                           float *global_scale, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * sharq_prepare_noalloc -- sharq_prepare for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, outputs and results, without
 * a workspace.  Its scratch (the NVFP4 per-row statistics) lives in a
 * 1 MiB device array inside the library, one per GPU, kept until the
 * process ends; the call itself allocates and frees nothing.
 *   - NVFP4 needs T <= SHARQ_NOALLOC_MAX_ROWS; more rows return
 *     SHARQ_ERR_WORKSPACE before any HIP call.  MXFP4 uses no scratch and
 *     takes any T that sharq_prepare takes.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (different streams, or host threads) race and give undefined
 *     results; calls ordered on one stream are safe.  The array's contents
 *     on entry do not matter.
 *   - The first call on a device looks up the array's device address with
 *     that device current (HIP errors there return SHARQ_ERR_HIP).
 */
#define SHARQ_NOALLOC_MAX_ROWS 65536
SHARQ_API sharq_status sharq_prepare_noalloc(const void *x, int32_t x_dtype, int64_t T, int64_t K, int64_t ldx,
                                   int32_t norm, const void *gamma, const void *beta, float eps,
                                   int32_t n, int32_t m, int32_t fmt, uint8_t *mask, uint8_t *b_codes,
                                   uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales,
                                   float *global_scale, void *stream);

/*
 * sharq_prepare_swiglu -- the fused preparation operator of sharq_prepare
 * (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
 * Inference, Abstract: mask generation and residual construction in one
 * operator) extended to the input of a SwiGLU down projection, SiLU(gate) *
 * up, computed straight from the gate/up product's FP32 output instead of a
 * stored bf16 activation (this fusion is not on the pages).  Per row t, for
 * k < K:
 *   xhat[k] = fl32(SiLU(gate[k]) * up[k]),  SiLU(g) = fl32(g / fl32(1 + e^-g))
 * with e^y a fixed sequence of correctly rounded float operations: Cody-Waite
 * reduction y = n*ln2 + r (n = rint(fl32(y*1.44269504)), ln2 split as
 * 0.693145752 + 1.42860677e-6), the degree-6 Taylor polynomial of e^r in
 * Horner form, times 2^n; 0 for y < -87, +inf for y > 88.  No
 * normalization; mask, backbone, residual and NVFP4 tensor scale exactly as
 * sharq_prepare.
 *
 *   gate_up      [T][ld] FP32, gate in columns [0, K), up in [K, 2K);
 *                16-byte aligned, ld >= 2K, ld*4 % 16 == 0
 *   other arguments and outputs as sharq_prepare (workspace:
 *   sharq_prepare_workspace_size())
 */
SHARQ_API sharq_status sharq_prepare_swiglu(const float *gate_up, int64_t T, int64_t K, int64_t ld,
                                  int32_t n, int32_t m, int32_t fmt, uint8_t *mask,
                                  uint8_t *b_codes, uint8_t *b_scales, uint8_t *r_codes,
                                  uint8_t *r_scales, float *global_scale, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Bytes of workspace sharq_quantize_weight needs. */
SHARQ_API size_t sharq_quantize_weight_workspace_size(int64_t experts, int64_t nout, int64_t K, int32_t fmt);

/*
 * sharq_quantize_weight -- the single FP4 weight payload that both paths
 * read (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract: one weight payload, a scale view per path).
 * Round-to-nearest-even quantization, run once per weight, offline.
 *
 *   w            [experts][nout][ldw] F16 or BF16 (PyTorch Linear layout,
 *                Y = X W^T): element k of row n of expert e at
 *                w[(e*nout + n)*ldw + k]; 16-byte aligned
 *   ldw          row stride in elements, ldw >= K, ldw*2 % 16 == 0
 *   codes        experts * nout*K/2 bytes: per expert (expert-major) the
 *                nout x K E2M1 codes, K-tiled with rows = nout
 *   scales       experts * nout*K/B bytes, per expert K-tiled likewise
 *   global_scale [experts] device floats: NVFP4 per-expert tensor scale
 *                amax/2688 (written); MXFP4: may be NULL, else 1.0f written
 *   workspace    sharq_quantize_weight_workspace_size() bytes
 */
SHARQ_API sharq_status sharq_quantize_weight(const void *w, int32_t w_dtype, int64_t experts, int64_t nout,
                                   int64_t K, int64_t ldw, int32_t fmt, uint8_t *codes, uint8_t *scales,
                                   float *global_scale, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * sharq_quantize_weight_gate_up -- sharq_quantize_weight for the gate/up
 * weight of a SwiGLU MLP, stored in the row order sharq_linear_swiglu
 * reads: w holds the gate rows in [0, nout/2) and the up rows in
 * [nout/2, nout) of every expert (the usual stacked layout); the payload
 * stores them interleaved in groups of 32 rows, payload row 64p + c = gate
 * row 32p + c and payload row 64p + 32 + c = up row 32p + c (c < 32).  Codes,
 * scales and tensor scales are those of sharq_quantize_weight of the
 * reordered rows.  nout % 64 == 0 (SHARQ_ERR_SHAPE otherwise); other
 * arguments, workspace and errors as sharq_quantize_weight.  (A layout of
 * this library, not of the pages.)
 */
SHARQ_API sharq_status sharq_quantize_weight_gate_up(const void *w, int32_t w_dtype, int64_t experts, int64_t nout,
                                           int64_t K, int64_t ldw, int32_t fmt, uint8_t *codes,
                                           uint8_t *scales, float *global_scale, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* Bytes of workspace sharq_linear needs for these arguments: 0, except for
 * MXFP4 products of one weight (experts == 1) with at most 64 rows that run
 * as independent products over equal K ranges summed in a fixed order
 * (decode batches with long K); then S * rows * nout floats of partial
 * products (S = 2, 4 or 8).  The value depends only on the arguments. */
SHARQ_API size_t sharq_linear_workspace_size(int64_t rows, int64_t K, int64_t nout, int64_t experts,
                                   int32_t fmt);

/*
 * sharq_linear -- the dual-path FP4 linear layer (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract: a sparse FP4
 * product on the backbone plus a dense FP4 product on the residual, which
 * restores what masking dropped and what backbone rounding lost).
 *
 *   Y[r][o] = sum_k ( deq(backbone)[src(r)][k] + deq(residual)[src(r)][k] )
 *                   * deq(W[e(r)])[o][k]
 * in FP32 accumulation (stored as FP32, or rounded to BF16 / F16), with
 * NVFP4 tensor scales applied as
 * x_global_scale * w_global_scale[e] in the epilogue.  Both paths read the
 * same weight codes and scales.  MXFP4 and NVFP4 multiply the backbone
 * densely on its zero-filled form (gfx950 has no block-scaled sparse FP4
 * matrix instruction); NVFP4_SP24 activations (weights in NVFP4) multiply
 * their compressed backbone with the 2:4 sparse f16 instruction on exactly
 * dequantized values.  The three give the same products up to the order of
 * the FP32 additions.
 *
 *   b_codes, b_scales, r_codes, r_scales  prepared activations, T rows,
 *                as written by sharq_prepare (K-tiled)
 *   x_global_scale  device float (NVFP4), NULL for MXFP4
 *   T, K         prepared rows and reduction length (K % 128 == 0); each
 *                operand (T*K/2 code bytes, one expert's nout*K/2) < 2 GiB
 *   w_codes, w_scales, w_global_scale  payload of sharq_quantize_weight
 *   experts, nout  weight shape
 *   group_offsets  experts == 1: NULL.  experts > 1: device int32
 *                [experts+1], non-decreasing, offsets[0] = 0,
 *                offsets[experts] = rows; output rows
 *                offsets[e]..offsets[e+1]-1 use expert e
 *   row_index    device int32 [rows] or NULL: output row r reads prepared row
 *                row_index[r] (0 <= row_index[r] < T); NULL reads row r
 *   rows         output rows (T when row_index is NULL and experts == 1)
 *   y            [rows][ldy] of y_dtype, ldy >= nout, aligned to its element
 *                size (vector stores of four elements are used when y is
 *                aligned to four elements and ldy % 4 == 0)
 *   y_dtype      SHARQ_F32 (the FP32 accumulator itself), SHARQ_BF16 or
 *                SHARQ_F16 (the FP32 accumulator rounded to nearest, ties
 *                to even, after the NVFP4 tensor scales; F16 overflows to
 *                infinity)
 *   workspace    sharq_linear_workspace_size() bytes of device memory,
 *                16-byte aligned (SHARQ_ERR_ALIGN otherwise),
 *                SHARQ_ERR_WORKSPACE when smaller; its contents on entry do
 *                not matter
 * Contents of group_offsets and row_index are trusted (device memory is not
 * read on the host); out-of-range values are undefined behaviour.  Every
 * output element is summed in a fixed order (no atomics), so repeated calls
 * on the same inputs give identical results.
 */
SHARQ_API sharq_status sharq_linear(const uint8_t *b_codes, const uint8_t *b_scales, const uint8_t *r_codes,
                          const uint8_t *r_scales, const float *x_global_scale, int64_t T,
                          int64_t K, int32_t fmt, const uint8_t *w_codes, const uint8_t *w_scales,
                          const float *w_global_scale, int64_t experts, int64_t nout,
                          const int32_t *group_offsets, const int32_t *row_index, int64_t rows,
                          void *y, int32_t y_dtype, int64_t ldy, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * sharq_linear_swiglu -- the dual-path FP4 product of a SwiGLU MLP's gate/up
 * linear with the preparation of the down projection's input fused into its
 * epilogue: the fused preparation operator (SharQ: Bridging Activation
 * Sparsity and FP4 Quantization for LLM Inference, Abstract: mask
 * generation and residual construction in one operator) applied to
 * SiLU(gate) * up while the FP32 product is still in registers, so neither
 * the product nor the activation goes through memory (this fusion is not on
 * the pages).  MXFP4 only.
 *
 * With Y the product sharq_linear computes (FP32, same accumulation order)
 * on a weight payload from sharq_quantize_weight_gate_up, and gate / up the
 * de-interleaved halves of each row of Y (gate[k] = Y[r][64(k/32) + k%32],
 * up[k] = Y[r][64(k/32) + 32 + k%32], k < nout/2), every output row r is
 * the sharq_prepare_swiglu preparation (same SiLU, same N:M selection, same
 * MXFP4 backbone and residual) of that row: an MXFP4 prepared activation of
 * rows x nout/2 elements.
 *
 *   b_codes .. rows  inputs as sharq_linear (activations MXFP4, weights from
 *                sharq_quantize_weight_gate_up; nout % 256 == 0)
 *   n, m         N:M mask of the output, 0 <= n <= m, m in {1, 2, 4}
 *                (m = 8 or 16: SHARQ_ERR_UNSUPPORTED)
 *   mask         [rows][nout/16] bitmap or NULL (not written), 4-byte aligned
 *   out_b_codes, out_b_scales, out_r_codes, out_r_scales  the prepared
 *                output, K-tiled with rows = rows and K = nout/2 (as
 *                sharq_prepare writes it); code arrays 8-byte aligned
 *   y            NULL, or [rows][ldy] FP32 (ldy >= nout, 4-byte aligned):
 *                also receives Y itself, in the interleaved column order
 * No workspace.  Validation and errors as sharq_linear.
 */
SHARQ_API sharq_status sharq_linear_swiglu(const uint8_t *b_codes, const uint8_t *b_scales, const uint8_t *r_codes,
                                 const uint8_t *r_scales, int64_t T, int64_t K, const uint8_t *w_codes,
                                 const uint8_t *w_scales, int64_t experts, int64_t nout,
                                 const int32_t *group_offsets, const int32_t *row_index, int64_t rows,
                                 int32_t n, int32_t m, uint8_t *mask, uint8_t *out_b_codes,
                                 uint8_t *out_b_scales, uint8_t *out_r_codes, uint8_t *out_r_scales, float *y,
                                 int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H */
