// Dual-path MXFP4 linear layer for gfx950.
//
// Source: SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract.  The backbone product (sparse
// path) and the residual product (dense path, which restores what masking
// dropped and what backbone rounding lost) read one FP4 weight payload.
//
// Y[m][n] = sum_k (Qb[m][k] + Qr[m][k]) * W[n][k], evaluated as two
// block-scaled FP4 matrix products into one FP32 accumulator: every weight
// fragment is read from LDS once and feeds the backbone MFMA and the
// residual MFMA (v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands and
// per-lane E8M0 scales).  The backbone is multiplied densely on its
// zero-filled form: gfx950's sparse matrix instructions (smfmac) take fp8,
// bf8, f16 or bf16 operands without block scales, so none holds MXFP4.
//
// Operand mapping for one 16x16x128 MFMA: the weight fragment is the A
// operand (16 weight rows), the activation fragment is the B operand (16
// token rows), so each lane's four accumulator values are four consecutive
// output columns of one token row and leave as one 128-bit store.  Lane l
// feeds row l%16 and the 32-element block l/16 of the 128-wide K step (16
// bytes of codes, one scale byte).
#include "device_util.h"
#include "kernels.h"

namespace sharq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kCbszFp4 = 4;  // MFMA operand format code for E2M1

__device__ __forceinline__ v4f mfma_fp4(v4i a, v4i b, v4f c, int sa, int sb) {
    const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    const v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, kCbszFp4, kCbszFp4, 0, sa, 0, sb);
}

template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_sel(v4i a, v4i b, v4f c, int sa, int sb) {
    const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    const v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, kCbszFp4, kCbszFp4, OPSEL, sa,
                                                           OPSEL, sb);
}

// ============================================================================
// Prefill: LDS-tiled, double-buffered.  Block tile BM token rows x BN weight
// rows, K step 128 (64 bytes of codes per row).  LDS row of 4 x 16-byte
// units, unit u of row r stored at u ^ ((r >> 2) & 3) so that the 16 rows
// read by one MFMA operand fetch hit disjoint banks.
// ============================================================================
constexpr int kKS = 128;          // K elements per stage
constexpr int kRowBytes = kKS / 2;  // 64 B of codes per row per stage

template <int BM, int BN>
struct StageLayout {
    static constexpr int W_CODES = 0;
    static constexpr int XB_CODES = W_CODES + BN * kRowBytes;
    static constexpr int XR_CODES = XB_CODES + BM * kRowBytes;
    static constexpr int W_SC = XR_CODES + BM * kRowBytes;
    static constexpr int XB_SC = W_SC + BN * 4;
    static constexpr int XR_SC = XB_SC + BM * 4;
    static constexpr int BYTES = XR_SC + BM * 4;
};

__device__ __forceinline__ int swz_unit(int row, int unit) { return unit ^ ((row >> 2) & 3); }

struct TileRows {
    int64_t m0;      // first output row of the tile
    int64_t m_end;   // one past the last valid output row
    int64_t expert;
};

// Map blockIdx.y to (expert, row range).  Dense: one expert.  Grouped: the
// tiles of expert e cover rows offsets[e]..offsets[e+1]-1 in BM-row steps.
template <int BM>
__device__ __forceinline__ bool tile_rows(const LinearArgs &a, int64_t tile, TileRows &tr) {
    if (a.offsets == nullptr) {
        tr.m0 = tile * BM;
        tr.m_end = a.rows;
        tr.expert = 0;
        return tr.m0 < a.rows;
    }
    int64_t acc = 0;
    for (int64_t e = 0; e < a.E; e++) {
        const int64_t lo = a.offsets[e], hi = a.offsets[e + 1];
        const int64_t nt = (hi - lo + BM - 1) / BM;
        if (tile < acc + nt) {
            tr.m0 = lo + (tile - acc) * BM;
            tr.m_end = hi;
            tr.expert = e;
            return true;
        }
        acc += nt;
    }
    return false;
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_dual_gemm_mx(LinearArgs a) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int FM = BM / WAVES_M / 16;  // token fragments per wave
    constexpr int FN = BN / WAVES_N / 16;  // weight fragments per wave
    using L = StageLayout<BM, BN>;
    constexpr int W_UNITS = BN * 4 / NT;   // 16-byte code units per thread per stage
    constexpr int X_UNITS = BM * 4 / NT;
    static_assert(BN * 4 % NT == 0 && BM * 4 % NT == 0, "tile / thread mismatch");
    static_assert(BN % NT == 0 || NT % BN == 0, "scale rows / thread mismatch");

    extern __shared__ __align__(16) uint8_t smem[];

    TileRows tr;
    if (!tile_rows<BM>(a, blockIdx.y, tr)) return;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t K = a.K;
    const int64_t kb = K / 2, ks = K / 32;  // code / scale bytes per row
    const uint8_t *wc = a.w_codes + tr.expert * a.nout * kb;
    const uint8_t *wsc = a.w_scales + tr.expert * a.nout * ks;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // ---- per-thread global sources (fixed across the K loop)
    const uint8_t *w_src[W_UNITS];
    const uint8_t *xb_src[X_UNITS], *xr_src[X_UNITS];
    int w_lds[W_UNITS], x_lds[X_UNITS];
#pragma unroll
    for (int i = 0; i < W_UNITS; i++) {
        const int u = tid + i * NT, row = u >> 2, unit = u & 3;
        const int64_t n = n0 + row;
        w_src[i] = n < a.nout ? wc + n * kb + unit * 16 : nullptr;
        w_lds[i] = row * kRowBytes + swz_unit(row, unit) * 16;
    }
#pragma unroll
    for (int i = 0; i < X_UNITS; i++) {
        const int u = tid + i * NT, row = u >> 2, unit = u & 3;
        const int64_t m = tr.m0 + row;
        if (m < tr.m_end) {
            const int64_t src = a.row_index ? (int64_t)a.row_index[m] : m;
            xb_src[i] = a.b_codes + src * kb + unit * 16;
            xr_src[i] = a.r_codes + src * kb + unit * 16;
        } else {
            xb_src[i] = xr_src[i] = nullptr;
        }
        x_lds[i] = row * kRowBytes + swz_unit(row, unit) * 16;
    }
    // scale dwords: thread t < BN loads weight row t, t < BM token row t
    const uint8_t *ws_src = nullptr, *xbs_src = nullptr, *xrs_src = nullptr;
    if (tid < BN && n0 + tid < a.nout) ws_src = wsc + (n0 + tid) * ks;
    if (tid < BM && tr.m0 + tid < tr.m_end) {
        const int64_t m = tr.m0 + tid;
        const int64_t src = a.row_index ? (int64_t)a.row_index[m] : m;
        xbs_src = a.b_scales + src * ks;
        xrs_src = a.r_scales + src * ks;
    }

    uint4 w_reg[W_UNITS], xb_reg[X_UNITS], xr_reg[X_UNITS];
    uint32_t ws_reg = 0x7F7F7F7Fu, xbs_reg = 0x7F7F7F7Fu, xrs_reg = 0x7F7F7F7Fu;
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    auto gload = [&](int64_t step) {
        const int64_t co = step * kRowBytes;
#pragma unroll
        for (int i = 0; i < W_UNITS; i++)
            w_reg[i] = w_src[i] ? *reinterpret_cast<const uint4 *>(w_src[i] + co) : zero4;
#pragma unroll
        for (int i = 0; i < X_UNITS; i++) {
            xb_reg[i] = xb_src[i] ? *reinterpret_cast<const uint4 *>(xb_src[i] + co) : zero4;
            xr_reg[i] = xr_src[i] ? *reinterpret_cast<const uint4 *>(xr_src[i] + co) : zero4;
        }
        const int64_t so = step * 4;
        if (ws_src) ws_reg = *reinterpret_cast<const uint32_t *>(ws_src + so);
        if (xbs_src) xbs_reg = *reinterpret_cast<const uint32_t *>(xbs_src + so);
        if (xrs_src) xrs_reg = *reinterpret_cast<const uint32_t *>(xrs_src + so);
    };
    auto lstore = [&](uint8_t *st) {
#pragma unroll
        for (int i = 0; i < W_UNITS; i++) *reinterpret_cast<uint4 *>(st + L::W_CODES + w_lds[i]) = w_reg[i];
#pragma unroll
        for (int i = 0; i < X_UNITS; i++) {
            *reinterpret_cast<uint4 *>(st + L::XB_CODES + x_lds[i]) = xb_reg[i];
            *reinterpret_cast<uint4 *>(st + L::XR_CODES + x_lds[i]) = xr_reg[i];
        }
        if (tid < BN) *reinterpret_cast<uint32_t *>(st + L::W_SC + tid * 4) = ws_reg;
        if (tid < BM) {
            *reinterpret_cast<uint32_t *>(st + L::XB_SC + tid * 4) = xbs_reg;
            *reinterpret_cast<uint32_t *>(st + L::XR_SC + tid * 4) = xrs_reg;
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int frow = lane & 15, fq = lane >> 4;
    const int64_t nsteps = K / kKS;

    gload(0);
    lstore(smem);
    __syncthreads();

    for (int64_t s = 0; s < nsteps; s++) {
        uint8_t *cur = smem + (s & 1) * L::BYTES;
        if (s + 1 < nsteps) gload(s + 1);

        v4i wf[FN];
        int wsf[FN];
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = wn * (FN * 16) + j * 16 + frow;
            wf[j] = *reinterpret_cast<const v4i *>(cur + L::W_CODES + row * kRowBytes + swz_unit(row, fq) * 16);
            wsf[j] = cur[L::W_SC + row * 4 + fq];
        }
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wm * (FM * 16) + i * 16 + frow;
            const int off = row * kRowBytes + swz_unit(row, fq) * 16;
            const v4i xb = *reinterpret_cast<const v4i *>(cur + L::XB_CODES + off);
            const v4i xr = *reinterpret_cast<const v4i *>(cur + L::XR_CODES + off);
            const int xbs = cur[L::XB_SC + row * 4 + fq];
            const int xrs = cur[L::XR_SC + row * 4 + fq];
#pragma unroll
            for (int j = 0; j < FN; j++) acc[i][j] = mfma_fp4(wf[j], xb, acc[i][j], wsf[j], xbs);
#pragma unroll
            for (int j = 0; j < FN; j++) acc[i][j] = mfma_fp4(wf[j], xr, acc[i][j], wsf[j], xrs);
        }
        if (s + 1 < nsteps) lstore(smem + ((s + 1) & 1) * L::BYTES);
        __syncthreads();
    }

    // ---- epilogue: lane holds Y[m][n..n+3]
#pragma unroll
    for (int i = 0; i < FM; i++) {
        const int64_t m = tr.m0 + wm * (FM * 16) + i * 16 + frow;
        if (m >= tr.m_end) continue;
        float *yrow = a.y + m * a.ldy;
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int64_t n = n0 + wn * (FN * 16) + j * 16 + fq * 4;
            const v4f v = acc[i][j];
            if (a.y_vec && n + 3 < a.nout) {
                *reinterpret_cast<v4f *>(yrow + n) = v;
            } else {
                if (n < a.nout) yrow[n] = v.x;
                if (n + 1 < a.nout) yrow[n + 1] = v.y;
                if (n + 2 < a.nout) yrow[n + 2] = v.z;
                if (n + 3 < a.nout) yrow[n + 3] = v.w;
            }
        }
    }
}

// ============================================================================
// Decode / small-T: no LDS.  Each wave owns 16 weight rows and a range of
// 512-element K chunks; lane (r = l%16, q = l/16) streams 64 contiguous code
// bytes and one scale dword of weight row r per chunk, so quarter q feeds
// blocks 4q..4q+3 and MFMA j (opsel j) uses block 4q+j.  Token rows come the
// same way (they are few and stay in L2).  With several K splits the partial
// sums meet in Y through FP32 atomic adds (Y zeroed first).
// ============================================================================
constexpr int kSmallWaves = 4;
constexpr int kChunkK = 512;

struct Chunk64 {
    uint4 u[4];
    uint32_t sc;
};

__device__ __forceinline__ void load_chunk(const uint8_t *codes_row, const uint8_t *sc_row, int64_t c,
                                           int q, int64_t K, bool valid, Chunk64 &o) {
    const int64_t k0 = c * kChunkK + q * 128;
    if (valid && k0 < K) {
        const uint4 *p = reinterpret_cast<const uint4 *>(codes_row + k0 / 2);
        o.u[0] = p[0]; o.u[1] = p[1]; o.u[2] = p[2]; o.u[3] = p[3];
        o.sc = *reinterpret_cast<const uint32_t *>(sc_row + k0 / 32);
    } else {
        o.u[0] = o.u[1] = o.u[2] = o.u[3] = make_uint4(0, 0, 0, 0);
        o.sc = 0x7F7F7F7Fu;
    }
}

__device__ __forceinline__ v4i as_v4i(uint4 u) { return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}; }

template <int FM>
__global__ __launch_bounds__(kSmallWaves * 64) void k_dual_gemm_mx_small(LinearArgs a, int64_t chunks_per_split,
                                                                          int atomic) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int64_t n0 = ((int64_t)blockIdx.x * kSmallWaves + wave) * 16;
    if (n0 >= a.nout) return;
    const int64_t K = a.K, kb = K / 2, ks = K / 32;
    const int64_t nch = (K + kChunkK - 1) / kChunkK;
    const int64_t c_begin = blockIdx.y * chunks_per_split;
    const int64_t c_end = min(nch, c_begin + chunks_per_split);

    const bool wvalid = n0 + r < a.nout;
    const uint8_t *wrow = a.w_codes + (n0 + r) * kb;
    const uint8_t *wsrow = a.w_scales + (n0 + r) * ks;
    const uint8_t *xb_row[FM], *xr_row[FM], *xbs_row[FM], *xrs_row[FM];
    bool xvalid[FM];
#pragma unroll
    for (int f = 0; f < FM; f++) {
        const int64_t m = f * 16 + r;
        xvalid[f] = m < a.rows;
        const int64_t src = xvalid[f] ? (a.row_index ? (int64_t)a.row_index[m] : m) : 0;
        xb_row[f] = a.b_codes + src * kb;
        xr_row[f] = a.r_codes + src * kb;
        xbs_row[f] = a.b_scales + src * ks;
        xrs_row[f] = a.r_scales + src * ks;
    }

    v4f acc[FM];
#pragma unroll
    for (int f = 0; f < FM; f++) acc[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t c = c_begin; c < c_end; c++) {
        Chunk64 w, xb[FM], xr[FM];
        load_chunk(wrow, wsrow, c, q, K, wvalid, w);
#pragma unroll
        for (int f = 0; f < FM; f++) {
            load_chunk(xb_row[f], xbs_row[f], c, q, K, xvalid[f], xb[f]);
            load_chunk(xr_row[f], xrs_row[f], c, q, K, xvalid[f], xr[f]);
        }
#pragma unroll
        for (int f = 0; f < FM; f++) {
            acc[f] = mfma_fp4_sel<0>(as_v4i(w.u[0]), as_v4i(xb[f].u[0]), acc[f], (int)w.sc, (int)xb[f].sc);
            acc[f] = mfma_fp4_sel<0>(as_v4i(w.u[0]), as_v4i(xr[f].u[0]), acc[f], (int)w.sc, (int)xr[f].sc);
            acc[f] = mfma_fp4_sel<1>(as_v4i(w.u[1]), as_v4i(xb[f].u[1]), acc[f], (int)w.sc, (int)xb[f].sc);
            acc[f] = mfma_fp4_sel<1>(as_v4i(w.u[1]), as_v4i(xr[f].u[1]), acc[f], (int)w.sc, (int)xr[f].sc);
            acc[f] = mfma_fp4_sel<2>(as_v4i(w.u[2]), as_v4i(xb[f].u[2]), acc[f], (int)w.sc, (int)xb[f].sc);
            acc[f] = mfma_fp4_sel<2>(as_v4i(w.u[2]), as_v4i(xr[f].u[2]), acc[f], (int)w.sc, (int)xr[f].sc);
            acc[f] = mfma_fp4_sel<3>(as_v4i(w.u[3]), as_v4i(xb[f].u[3]), acc[f], (int)w.sc, (int)xb[f].sc);
            acc[f] = mfma_fp4_sel<3>(as_v4i(w.u[3]), as_v4i(xr[f].u[3]), acc[f], (int)w.sc, (int)xr[f].sc);
        }
    }
#pragma unroll
    for (int f = 0; f < FM; f++) {
        const int64_t m = f * 16 + r;
        if (m >= a.rows) continue;
        float *yrow = a.y + m * a.ldy;
        const int64_t n = n0 + q * 4;
        const float vals[4] = {acc[f].x, acc[f].y, acc[f].z, acc[f].w};
        if (atomic) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (n + i < a.nout) atomicAdd(yrow + n + i, vals[i]);
        } else if (a.y_vec && n + 3 < a.nout) {
            *reinterpret_cast<v4f *>(yrow + n) = acc[f];
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (n + i < a.nout) yrow[n + i] = vals[i];
        }
    }
}

__global__ void k_zero_rows(float *y, int64_t rows, int64_t cols, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < rows * cols) y[(i / cols) * ldy + i % cols] = 0.0f;
}

// ============================================================================
// launcher
// ============================================================================
template <int BM, int BN, int WM, int WN>
static hipError_t launch_prefill(const LinearArgs &a, hipStream_t st) {
    using L = StageLayout<BM, BN>;
    const size_t lds = 2 * (size_t)L::BYTES;
    static bool attr_set = false;  // idempotent; benign if two threads race to set it
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_dual_gemm_mx<BM, BN, WM, WN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    int64_t mtiles;
    if (a.offsets) mtiles = (a.rows + BM - 1) / BM + a.E;  // upper bound; extra blocks exit
    else mtiles = (a.rows + BM - 1) / BM;
    const dim3 grid((unsigned)((a.nout + BN - 1) / BN), (unsigned)mtiles);
    hipLaunchKernelGGL((k_dual_gemm_mx<BM, BN, WM, WN>), grid, dim3(WM * WN * 64), lds, st, a);
    return hipGetLastError();
}

template <int FM>
static hipError_t launch_small(const LinearArgs &a, hipStream_t st) {
    const int64_t nwaves_n = (a.nout + 15) / 16;
    const int64_t nch = (a.K + kChunkK - 1) / kChunkK;
    // aim for ~8 waves per CU on 256 CUs
    int64_t split = (2048 + nwaves_n - 1) / nwaves_n;
    if (split > nch) split = nch;
    if (split < 1) split = 1;
    const int64_t cps = (nch + split - 1) / split;
    split = (nch + cps - 1) / cps;
    const int atomic = split > 1;
    if (atomic) {
        const int64_t n = a.rows * a.nout;
        hipLaunchKernelGGL(k_zero_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.y, a.rows,
                           a.nout, a.ldy);
    }
    const dim3 grid((unsigned)((nwaves_n + kSmallWaves - 1) / kSmallWaves), (unsigned)split);
    hipLaunchKernelGGL((k_dual_gemm_mx_small<FM>), grid, dim3(kSmallWaves * 64), 0, st, a, cps, atomic);
    return hipGetLastError();
}

hipError_t launch_linear_mx(const LinearArgs &a, hipStream_t st) {
    if (a.offsets == nullptr && a.rows <= 64) {
        if (a.rows <= 16) return launch_small<1>(a, st);
        if (a.rows <= 32) return launch_small<2>(a, st);
        if (a.rows <= 48) return launch_small<3>(a, st);
        return launch_small<4>(a, st);
    }
    if (a.offsets) return launch_prefill<128, 256, 2, 2>(a, st);
    return launch_prefill<256, 256, 2, 2>(a, st);
}

}  // namespace sharq
