// C ABI of the SharQ hot path (declared in include/sharq.h): host-side
// argument validation and dispatch to the gfx950 kernels.  Every check runs
// before the first HIP call, so invalid arguments are rejected without
// touching the GPU (and are testable on machines without one).
#include "../../include/sharq.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "kernels.h"

using namespace sharq;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// the normalized MXFP4 prep launches one workgroup per row
constexpr int64_t kMaxPrepRows = ((int64_t)1 << 31) - 64;
static_assert(SHARQ_NOALLOC_MAX_ROWS == kNoallocRows, "header and library agree on the scratch size");

int block_of(int32_t fmt) { return fmt == SHARQ_MXFP4 ? 32 : 16; }

bool valid_fmt(int32_t fmt) { return fmt == SHARQ_MXFP4 || fmt == SHARQ_NVFP4 || fmt == SHARQ_NVFP4_SP24; }

bool is_nv(int32_t fmt) { return fmt == SHARQ_NVFP4 || fmt == SHARQ_NVFP4_SP24; }

// quantization format of the kernels (the compressed backbone is a store
// option of NVFP4)
int kernel_fmt(int32_t fmt) { return fmt == SHARQ_MXFP4 ? kFmtMx : kFmtNv; }

// NVFP4_SP24 preparation: the 2:4 mask, whole K tiles and 32-bit store
// offsets (the compressed store path)
sharq_status sp24_shape(int32_t fmt, int64_t T, int64_t K, int32_t n, int32_t m) {
    if (fmt != SHARQ_NVFP4_SP24) return SHARQ_OK;
    if (n != 2 || m != 4) return SHARQ_ERR_NM;
    if (K % 128 != 0 || T * (K / 2) >= ((int64_t)1 << 32)) return SHARQ_ERR_SHAPE;
    return SHARQ_OK;
}

// hipError_t of this thread's most recent entry-point call that reached HIP.
thread_local int g_last_hip_error = 0;

bool debug_mode() {
    const char *v = std::getenv("SHARQ_DEBUG");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
}

// Status of an entry point's launches on `st`.  With SHARQ_DEBUG=1 the call
// also waits for them (unless the stream is being captured into a graph, where
// waiting is not allowed) and reports any error the kernels raised, naming the
// entry point on stderr.
sharq_status finish(const char *what, hipError_t e, hipStream_t st) {
    const bool debug = debug_mode();
    if (e == hipSuccess && debug) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(st, &cs);
        if (e == hipSuccess && cs == hipStreamCaptureStatusNone) {
            e = hipStreamSynchronize(st);
            if (e == hipSuccess) e = hipGetLastError();
        }
    }
    g_last_hip_error = (int)e;
    if (e == hipSuccess) return SHARQ_OK;
    if (debug) std::fprintf(stderr, "sharq: %s: %s\n", what, hipGetErrorString(e));
    return SHARQ_ERR_HIP;
}

}  // namespace

extern "C" {

int sharq_abi_version(void) { return SHARQ_ABI_VERSION; }

int sharq_last_hip_error(void) { return g_last_hip_error; }

const char *sharq_status_string(int status) {
    switch (status) {
        case SHARQ_OK: return "ok";
        case SHARQ_ERR_NULL: return "required pointer is NULL";
        case SHARQ_ERR_SHAPE: return "invalid shape or leading dimension";
        case SHARQ_ERR_NM: return "invalid N:M pattern";
        case SHARQ_ERR_DTYPE: return "unsupported element type";
        case SHARQ_ERR_ALIGN: return "pointer or stride not aligned";
        case SHARQ_ERR_WORKSPACE: return "workspace missing or too small (or more rows than the built-in scratch holds)";
        case SHARQ_ERR_UNSUPPORTED: return "unsupported format or combination";
        case SHARQ_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

size_t sharq_prepare_workspace_size(int64_t T, int64_t K, int32_t fmt) {
    (void)K;
    return prepare_workspace_bytes(T, kernel_fmt(fmt));
}

}  // extern "C"

namespace {

// Argument checks of sharq_prepare and sharq_prepare_noalloc, before any HIP
// call, and the kernel arguments they describe.  need_ws: check the caller's
// workspace (sharq_prepare) or the built-in scratch limit (noalloc).
sharq_status prepare_args(const void *x, int32_t x_dtype, int64_t T, int64_t K, int64_t ldx, int32_t norm,
                          const void *gamma, const void *beta, float eps, int32_t n, int32_t m, int32_t fmt,
                          uint8_t *mask, uint8_t *b_codes, uint8_t *b_scales, uint8_t *r_codes,
                          uint8_t *r_scales, float *global_scale, bool need_ws, void *workspace,
                          size_t workspace_bytes, PrepArgs &a) {
    if (!valid_fmt(fmt)) return SHARQ_ERR_UNSUPPORTED;
    if (x_dtype != SHARQ_BF16 && x_dtype != SHARQ_F16) return SHARQ_ERR_DTYPE;
    if (norm != SHARQ_NORM_NONE && norm != SHARQ_NORM_RMS && norm != SHARQ_NORM_LAYER)
        return SHARQ_ERR_UNSUPPORTED;
    if (T < 0 || K <= 0 || ldx < K || K % block_of(fmt) != 0) return SHARQ_ERR_SHAPE;
    if (T >= kMaxPrepRows) return SHARQ_ERR_SHAPE;  // one workgroup per row must fit the grid
    if (m != 1 && m != 2 && m != 4 && m != 8 && m != 16) return SHARQ_ERR_NM;
    if (n < 0 || n > m || K % m != 0) return SHARQ_ERR_NM;
    if (const sharq_status sp = sp24_shape(fmt, T, K, n, m); sp != SHARQ_OK) return sp;
    if (T == 0) return SHARQ_OK;
    if (!x || !b_codes || !b_scales || !r_codes || !r_scales) return SHARQ_ERR_NULL;
    if (norm != SHARQ_NORM_NONE && !gamma) return SHARQ_ERR_NULL;
    if (is_nv(fmt) && !global_scale) return SHARQ_ERR_NULL;
    if (!aligned(x, 16) || (ldx * 2) % 16 != 0) return SHARQ_ERR_ALIGN;
    if ((gamma && !aligned(gamma, 16)) || (beta && !aligned(beta, 16))) return SHARQ_ERR_ALIGN;
    if (!aligned(b_codes, 4) || !aligned(r_codes, 4)) return SHARQ_ERR_ALIGN;
    if (global_scale && !aligned(global_scale, 4)) return SHARQ_ERR_ALIGN;
    if (need_ws) {
        const size_t need = prepare_workspace_bytes(T, kernel_fmt(fmt));
        if (need > 0 && (!workspace || workspace_bytes < need)) return SHARQ_ERR_WORKSPACE;
        if (need > 0 && !aligned(workspace, 16)) return SHARQ_ERR_ALIGN;
    } else if (is_nv(fmt) && T > kNoallocRows) {
        return SHARQ_ERR_WORKSPACE;  // more rows than the built-in scratch holds
    }

    a = PrepArgs{};
    a.x = static_cast<const uint16_t *>(x);
    a.T = T;
    a.K = K;
    a.ldx = ldx;
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.beta = norm == SHARQ_NORM_LAYER ? static_cast<const uint16_t *>(beta) : nullptr;
    a.eps = eps;
    a.n = n;
    a.m = m;
    a.norm = norm;
    a.fmt = kernel_fmt(fmt);
    a.sp = fmt == SHARQ_NVFP4_SP24;
    a.bf16 = x_dtype == SHARQ_BF16;
    a.mask = mask;
    a.b_codes = b_codes;
    a.b_scales = b_scales;
    a.r_codes = r_codes;
    a.r_scales = r_scales;
    a.global_scale = global_scale;
    a.off32 = K % 128 == 0 && T * (K / 2) < ((int64_t)1 << 32);
    return SHARQ_OK;
}

}  // namespace

extern "C" {

sharq_status sharq_prepare(const void *x, int32_t x_dtype, int64_t T, int64_t K, int64_t ldx,
                           int32_t norm, const void *gamma, const void *beta, float eps, int32_t n,
                           int32_t m, int32_t fmt, uint8_t *mask, uint8_t *b_codes, uint8_t *b_scales,
                           uint8_t *r_codes, uint8_t *r_scales, float *global_scale, void *workspace,
                           size_t workspace_bytes, void *stream) {
    PrepArgs a{};
    const sharq_status s = prepare_args(x, x_dtype, T, K, ldx, norm, gamma, beta, eps, n, m, fmt, mask, b_codes,
                                        b_scales, r_codes, r_scales, global_scale, true, workspace,
                                        workspace_bytes, a);
    if (s != SHARQ_OK || T == 0) return s;
    return finish("sharq_prepare", launch_prepare(a, workspace, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

sharq_status sharq_prepare_noalloc(const void *x, int32_t x_dtype, int64_t T, int64_t K, int64_t ldx,
                                   int32_t norm, const void *gamma, const void *beta, float eps, int32_t n,
                                   int32_t m, int32_t fmt, uint8_t *mask, uint8_t *b_codes,
                                   uint8_t *b_scales, uint8_t *r_codes, uint8_t *r_scales,
                                   float *global_scale, void *stream) {
    PrepArgs a{};
    const sharq_status s = prepare_args(x, x_dtype, T, K, ldx, norm, gamma, beta, eps, n, m, fmt, mask, b_codes,
                                        b_scales, r_codes, r_scales, global_scale, false, nullptr, 0, a);
    if (s != SHARQ_OK || T == 0) return s;
    return finish("sharq_prepare_noalloc", launch_prepare_noalloc(a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

sharq_status sharq_prepare_swiglu(const float *gate_up, int64_t T, int64_t K, int64_t ld, int32_t n, int32_t m,
                                  int32_t fmt, uint8_t *mask, uint8_t *b_codes, uint8_t *b_scales,
                                  uint8_t *r_codes, uint8_t *r_scales, float *global_scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (!valid_fmt(fmt)) return SHARQ_ERR_UNSUPPORTED;
    if (T < 0 || K <= 0 || ld < 2 * K || K % block_of(fmt) != 0) return SHARQ_ERR_SHAPE;
    if (T >= kMaxPrepRows) return SHARQ_ERR_SHAPE;
    if (m != 1 && m != 2 && m != 4 && m != 8 && m != 16) return SHARQ_ERR_NM;
    if (n < 0 || n > m || K % m != 0) return SHARQ_ERR_NM;
    if (const sharq_status sp = sp24_shape(fmt, T, K, n, m); sp != SHARQ_OK) return sp;
    if (T == 0) return SHARQ_OK;
    if (!gate_up || !b_codes || !b_scales || !r_codes || !r_scales) return SHARQ_ERR_NULL;
    if (is_nv(fmt) && !global_scale) return SHARQ_ERR_NULL;
    if (!aligned(gate_up, 16) || (ld * 4) % 16 != 0) return SHARQ_ERR_ALIGN;
    if (!aligned(b_codes, 4) || !aligned(r_codes, 4)) return SHARQ_ERR_ALIGN;
    if (global_scale && !aligned(global_scale, 4)) return SHARQ_ERR_ALIGN;
    const size_t need = prepare_workspace_bytes(T, kernel_fmt(fmt));
    if (need > 0 && (!workspace || workspace_bytes < need)) return SHARQ_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return SHARQ_ERR_ALIGN;

    PrepArgs a{};
    a.T = T;
    a.K = K;
    a.n = n;
    a.m = m;
    a.norm = SHARQ_NORM_NONE;
    a.fmt = kernel_fmt(fmt);
    a.sp = fmt == SHARQ_NVFP4_SP24;
    a.mask = mask;
    a.b_codes = b_codes;
    a.b_scales = b_scales;
    a.r_codes = r_codes;
    a.r_scales = r_scales;
    a.global_scale = global_scale;
    a.off32 = K % 128 == 0 && T * (K / 2) < ((int64_t)1 << 32);
    a.gu = gate_up;
    a.ldgu = ld;
    return finish("sharq_prepare_swiglu", launch_prepare_swiglu(a, workspace, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

size_t sharq_quantize_weight_workspace_size(int64_t experts, int64_t nout, int64_t K, int32_t fmt) {
    (void)K;
    return quantize_weight_workspace_bytes(experts, nout, kernel_fmt(fmt));
}

}  // extern "C"

namespace {

sharq_status quantize_weight_impl(const char *what, bool interleave, const void *w, int32_t w_dtype,
                                  int64_t experts, int64_t nout, int64_t K, int64_t ldw, int32_t fmt,
                                  uint8_t *codes, uint8_t *scales, float *global_scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (!valid_fmt(fmt)) return SHARQ_ERR_UNSUPPORTED;
    if (w_dtype != SHARQ_BF16 && w_dtype != SHARQ_F16) return SHARQ_ERR_DTYPE;
    if (experts < 1 || nout < 0 || K <= 0 || K % block_of(fmt) != 0 || ldw < K) return SHARQ_ERR_SHAPE;
    if (interleave && nout % 64 != 0) return SHARQ_ERR_SHAPE;
    if (nout == 0) return SHARQ_OK;
    if (!w || !codes || !scales) return SHARQ_ERR_NULL;
    if (is_nv(fmt) && !global_scale) return SHARQ_ERR_NULL;
    if (!aligned(w, 16) || (ldw * 2) % 16 != 0 || !aligned(codes, 4) ||
        (global_scale && !aligned(global_scale, 4)))
        return SHARQ_ERR_ALIGN;
    const size_t need = quantize_weight_workspace_bytes(experts, nout, kernel_fmt(fmt));
    if (need > 0 && (!workspace || workspace_bytes < need)) return SHARQ_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return SHARQ_ERR_ALIGN;
    QuantWArgs a;
    a.w = static_cast<const uint16_t *>(w);
    a.E = experts;
    a.nout = nout;
    a.K = K;
    a.ldw = ldw;
    a.fmt = kernel_fmt(fmt);
    a.bf16 = w_dtype == SHARQ_BF16;
    a.codes = codes;
    a.scales = scales;
    a.global_scale = global_scale;
    a.gate_up_interleave = interleave;
    return finish(what, launch_quantize_weight(a, workspace, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

sharq_status sharq_quantize_weight(const void *w, int32_t w_dtype, int64_t experts, int64_t nout,
                                   int64_t K, int64_t ldw, int32_t fmt, uint8_t *codes, uint8_t *scales,
                                   float *global_scale, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    return quantize_weight_impl("sharq_quantize_weight", false, w, w_dtype, experts, nout, K, ldw, fmt, codes,
                                scales, global_scale, workspace, workspace_bytes, stream);
}

sharq_status sharq_quantize_weight_gate_up(const void *w, int32_t w_dtype, int64_t experts, int64_t nout,
                                           int64_t K, int64_t ldw, int32_t fmt, uint8_t *codes,
                                           uint8_t *scales, float *global_scale, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    return quantize_weight_impl("sharq_quantize_weight_gate_up", true, w, w_dtype, experts, nout, K, ldw, fmt,
                                codes, scales, global_scale, workspace, workspace_bytes, stream);
}

size_t sharq_linear_workspace_size(int64_t rows, int64_t K, int64_t nout, int64_t experts,
                                   int32_t fmt) {
    return linear_workspace_bytes(rows, K, nout, experts, fmt);
}

sharq_status sharq_linear(const uint8_t *b_codes, const uint8_t *b_scales, const uint8_t *r_codes,
                          const uint8_t *r_scales, const float *x_global_scale, int64_t T, int64_t K,
                          int32_t fmt, const uint8_t *w_codes, const uint8_t *w_scales,
                          const float *w_global_scale, int64_t experts, int64_t nout,
                          const int32_t *group_offsets, const int32_t *row_index, int64_t rows,
                          void *y, int32_t y_dtype, int64_t ldy, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (!valid_fmt(fmt)) return SHARQ_ERR_UNSUPPORTED;
    if (y_dtype != SHARQ_F32 && y_dtype != SHARQ_BF16 && y_dtype != SHARQ_F16) return SHARQ_ERR_DTYPE;
    if (T < 0 || K <= 0 || K % 128 != 0 || experts < 1 || nout < 0 || rows < 0 || ldy < nout)
        return SHARQ_ERR_SHAPE;
    if (experts == 1 && !group_offsets && !row_index && rows != T) return SHARQ_ERR_SHAPE;
    if (experts > 1 && !group_offsets) return SHARQ_ERR_NULL;
    if (rows == 0 || nout == 0) return SHARQ_OK;
    if (T == 0) return SHARQ_ERR_SHAPE;  // rows to produce but nothing to read
    if (!b_codes || !b_scales || !r_codes || !r_scales || !w_codes || !w_scales || !y)
        return SHARQ_ERR_NULL;
    if (is_nv(fmt) && (!x_global_scale || !w_global_scale)) return SHARQ_ERR_NULL;
    if (!aligned(b_codes, 16) || !aligned(r_codes, 16) || !aligned(w_codes, 16) ||
        !aligned(b_scales, 4) || !aligned(r_scales, 4) || !aligned(w_scales, 4))
        return SHARQ_ERR_ALIGN;
    const size_t ysize = y_dtype == SHARQ_F32 ? 4 : 2;
    if (!aligned(y, ysize)) return SHARQ_ERR_ALIGN;
    // operands are addressed with 32-bit buffer offsets
    const int64_t limit = (int64_t)1 << 31;
    if (T * (K / 2) >= limit || nout * (K / 2) >= limit) return SHARQ_ERR_SHAPE;
    const int kfmt = fmt == SHARQ_MXFP4 ? kFmtMx : (fmt == SHARQ_NVFP4 ? kFmtNv : kFmtNvSp);
    const size_t need = linear_workspace_bytes(rows, K, nout, experts, kfmt);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SHARQ_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return SHARQ_ERR_ALIGN;
    LinearArgs a;
    a.b_codes = b_codes;
    a.b_scales = b_scales;
    a.r_codes = r_codes;
    a.r_scales = r_scales;
    a.x_gscale = x_global_scale;
    a.T = T;
    a.K = K;
    a.fmt = kfmt;
    a.w_codes = w_codes;
    a.w_scales = w_scales;
    a.w_gscale = w_global_scale;
    a.E = experts;
    a.nout = nout;
    a.offsets = experts > 1 ? group_offsets : nullptr;
    a.row_index = row_index;
    a.rows = rows;
    a.y = y;
    a.ydt = y_dtype == SHARQ_F32 ? kOutF32 : (y_dtype == SHARQ_BF16 ? kOutBf16 : kOutF16);
    a.ldy = ldy;
    a.y_vec = aligned(y, 4 * ysize) && ldy % 4 == 0;
    a.ksplit_tiles = 0;
    a.split_stride = 0;
    a.xcd_band = 0;
    a.p_mask = a.p_b_codes = a.p_b_scales = a.p_r_codes = a.p_r_scales = nullptr;
    a.p_n = a.p_m = 0;
    return finish("sharq_linear", launch_linear(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

sharq_status sharq_linear_swiglu(const uint8_t *b_codes, const uint8_t *b_scales, const uint8_t *r_codes,
                                 const uint8_t *r_scales, int64_t T, int64_t K, const uint8_t *w_codes,
                                 const uint8_t *w_scales, int64_t experts, int64_t nout,
                                 const int32_t *group_offsets, const int32_t *row_index, int64_t rows,
                                 int32_t n, int32_t m, uint8_t *mask, uint8_t *out_b_codes,
                                 uint8_t *out_b_scales, uint8_t *out_r_codes, uint8_t *out_r_scales, float *y,
                                 int64_t ldy, void *stream) {
    if (T < 0 || K <= 0 || K % 128 != 0 || experts < 1 || nout < 0 || nout % 256 != 0 || rows < 0)
        return SHARQ_ERR_SHAPE;
    if (m != 1 && m != 2 && m != 4 && m != 8 && m != 16) return SHARQ_ERR_NM;
    if (n < 0 || n > m) return SHARQ_ERR_NM;
    if (m > 4) return SHARQ_ERR_UNSUPPORTED;  // mask groups held inside one lane
    if (experts == 1 && !group_offsets && !row_index && rows != T) return SHARQ_ERR_SHAPE;
    if (experts > 1 && !group_offsets) return SHARQ_ERR_NULL;
    if (y && ldy < nout) return SHARQ_ERR_SHAPE;
    if (rows == 0 || nout == 0) return SHARQ_OK;
    if (T == 0) return SHARQ_ERR_SHAPE;
    if (!b_codes || !b_scales || !r_codes || !r_scales || !w_codes || !w_scales || !out_b_codes ||
        !out_b_scales || !out_r_codes || !out_r_scales)
        return SHARQ_ERR_NULL;
    if (!aligned(b_codes, 16) || !aligned(r_codes, 16) || !aligned(w_codes, 16) || !aligned(b_scales, 4) ||
        !aligned(r_scales, 4) || !aligned(w_scales, 4) || !aligned(out_b_codes, 8) || !aligned(out_r_codes, 8) ||
        (mask && !aligned(mask, 4)) || (y && !aligned(y, 4)))
        return SHARQ_ERR_ALIGN;
    const int64_t limit = (int64_t)1 << 31;
    if (T * (K / 2) >= limit || nout * (K / 2) >= limit) return SHARQ_ERR_SHAPE;
    LinearArgs a;
    a.b_codes = b_codes;
    a.b_scales = b_scales;
    a.r_codes = r_codes;
    a.r_scales = r_scales;
    a.x_gscale = nullptr;
    a.T = T;
    a.K = K;
    a.fmt = kFmtMx;
    a.w_codes = w_codes;
    a.w_scales = w_scales;
    a.w_gscale = nullptr;
    a.E = experts;
    a.nout = nout;
    a.offsets = experts > 1 ? group_offsets : nullptr;
    a.row_index = row_index;
    a.rows = rows;
    a.y = y;
    a.ydt = kOutF32;
    a.ldy = y ? ldy : nout;
    a.y_vec = y && aligned(y, 16) && ldy % 4 == 0;
    a.ksplit_tiles = 0;
    a.split_stride = 0;
    a.xcd_band = 0;
    a.p_mask = mask;
    a.p_b_codes = out_b_codes;
    a.p_b_scales = out_b_scales;
    a.p_r_codes = out_r_codes;
    a.p_r_scales = out_r_scales;
    a.p_n = n;
    a.p_m = m;
    return finish("sharq_linear_swiglu", launch_linear_swiglu(a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream));
}

}  // extern "C"
