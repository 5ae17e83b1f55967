// Dual-path NVFP4 linear layer for gfx950, and the linear-layer dispatcher.
//
// NVFP4 elements carry an E4M3 scale per 16 values.  gfx950's block-scaled
// matrix instruction takes one power-of-two (E8M0) scale per 32 values, and
// an E2M1 value times an E4M3 scale needs up to 6 significant bits, so no
// FP4/FP6/FP8 operand holds it exactly; bf16 does.  The kernel therefore
// dequantizes code*scale into bf16 registers on the LDS -> register path and
// runs v_mfma_f32_16x16x32_bf16, with the two tensor scales (activation and
// weight) applied to the FP32 accumulator in the epilogue.  Staging, tile
// mapping and the shared weight fragment per backbone/residual pair follow
// the MXFP4 kernel.
#include "device_util.h"
#include "kernels.h"

namespace sharq {

hipError_t launch_linear_mx(const LinearArgs &a, hipStream_t st);

typedef float v4f_nv __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kNvKS = 128;           // K per stage
constexpr int kNvRow = kNvKS / 2;    // 64 B of codes per row per stage
constexpr int kNvScRow = kNvKS / 16; // 8 E4M3 scale bytes per row per stage

template <int BM, int BN>
struct NvStage {
    static constexpr int W_CODES = 0;
    static constexpr int XB_CODES = W_CODES + BN * kNvRow;
    static constexpr int XR_CODES = XB_CODES + BM * kNvRow;
    static constexpr int W_SC = XR_CODES + BM * kNvRow;
    static constexpr int XB_SC = W_SC + BN * kNvScRow;
    static constexpr int XR_SC = XB_SC + BM * kNvScRow;
    static constexpr int BYTES = XR_SC + BM * kNvScRow;
};

__device__ __forceinline__ int nv_swz(int row, int unit) { return unit ^ ((row >> 2) & 3); }

// bf16 bit pattern of the E2M1 code (low 4 bits of c) times s (an E4M3 value,
// so the product has at most 6 significant bits and is exact in bf16).
__device__ __forceinline__ uint32_t e2m1_times_bf16(uint32_t c, float s) {
    const uint32_t m = c & 7u;
    const uint32_t mag = m == 0u ? 0u : (m == 1u ? 0x3F000000u : ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22)));
    const float v = __fmul_rn(__uint_as_float(mag | ((c & 8u) << 28)), s);
    return __float_as_uint(v) >> 16;
}

// Eight codes (one 32-bit word, element i in nibble i) -> eight bf16 values.
__device__ __forceinline__ v8bf dequant8(uint32_t w, float s) {
    v4u r;
    r.x = e2m1_times_bf16(w, s) | (e2m1_times_bf16(w >> 4, s) << 16);
    r.y = e2m1_times_bf16(w >> 8, s) | (e2m1_times_bf16(w >> 12, s) << 16);
    r.z = e2m1_times_bf16(w >> 16, s) | (e2m1_times_bf16(w >> 20, s) << 16);
    r.w = e2m1_times_bf16(w >> 24, s) | (e2m1_times_bf16(w >> 28, s) << 16);
    return __builtin_bit_cast(v8bf, r);
}

template <int BM>
__device__ __forceinline__ bool nv_tile_rows(const LinearArgs &a, int64_t tile, int64_t &m0, int64_t &m_end,
                                             int64_t &expert) {
    if (a.offsets == nullptr) {
        m0 = tile * BM;
        m_end = a.rows;
        expert = 0;
        return m0 < a.rows;
    }
    int64_t acc = 0;
    for (int64_t e = 0; e < a.E; e++) {
        const int64_t lo = a.offsets[e], hi = a.offsets[e + 1];
        const int64_t nt = (hi - lo + BM - 1) / BM;
        if (tile < acc + nt) {
            m0 = lo + (tile - acc) * BM;
            m_end = hi;
            expert = e;
            return true;
        }
        acc += nt;
    }
    return false;
}

// Lane (row, q) of a fragment covers, in K sub-step t (0..3) of a stage, the
// eight elements 32q + 8t .. +8 (the same permutation of K for both operands),
// so each lane reads one 16-byte unit of codes per fragment per stage and the
// two scale bytes 2q, 2q+1.
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_dual_gemm_nv(LinearArgs a) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int FM = BM / WAVES_M / 16;
    constexpr int FN = BN / WAVES_N / 16;
    using L = NvStage<BM, BN>;
    constexpr int W_UNITS = BN * 4 / NT;
    constexpr int X_UNITS = BM * 4 / NT;
    static_assert(BN * 4 % NT == 0 && BM * 4 % NT == 0, "tile / thread mismatch");

    extern __shared__ __align__(16) uint8_t smem[];
    int64_t m0, m_end, expert;
    if (!nv_tile_rows<BM>(a, blockIdx.y, m0, m_end, expert)) return;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t K = a.K, kb = K / 2, ks = K / 16;
    const uint8_t *wc = a.w_codes + expert * a.nout * kb;
    const uint8_t *wsc = a.w_scales + expert * a.nout * ks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // K-tiled operands: a stage is one tile of rows x 64 code bytes and
    // rows x 8 scale bytes; the tile stride is the array's row count
    const int64_t tw = a.nout, tx = a.T;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const uint8_t *w_src[W_UNITS];
    const uint8_t *xb_src[X_UNITS], *xr_src[X_UNITS];
    int w_lds[W_UNITS], x_lds[X_UNITS];
#pragma unroll
    for (int i = 0; i < W_UNITS; i++) {
        const int u = tid + i * NT, row = u >> 2, unit = u & 3;
        const int64_t n = n0 + row;
        w_src[i] = n < a.nout ? wc + n * kNvRow + unit * 16 : nullptr;
        w_lds[i] = row * kNvRow + nv_swz(row, unit) * 16;
    }
#pragma unroll
    for (int i = 0; i < X_UNITS; i++) {
        const int u = tid + i * NT, row = u >> 2, unit = u & 3;
        const int64_t m = m0 + row;
        if (m < m_end) {
            const int64_t src = a.row_index ? (int64_t)a.row_index[m] : m;
            xb_src[i] = a.b_codes + src * kNvRow + unit * 16;
            xr_src[i] = a.r_codes + src * kNvRow + unit * 16;
        } else {
            xb_src[i] = xr_src[i] = nullptr;
        }
        x_lds[i] = row * kNvRow + nv_swz(row, unit) * 16;
    }
    // scales: 8 bytes per row per stage; thread t handles row t (if present)
    const uint8_t *ws_src = nullptr, *xbs_src = nullptr, *xrs_src = nullptr;
    if (tid < BN && n0 + tid < a.nout) ws_src = wsc + (n0 + tid) * kNvScRow;
    if (tid < BM && m0 + tid < m_end) {
        const int64_t m = m0 + tid;
        const int64_t src = a.row_index ? (int64_t)a.row_index[m] : m;
        xbs_src = a.b_scales + src * kNvScRow;
        xrs_src = a.r_scales + src * kNvScRow;
    }
    uint4 w_reg[W_UNITS], xb_reg[X_UNITS], xr_reg[X_UNITS];
    uint2 ws_reg = make_uint2(0, 0), xbs_reg = make_uint2(0, 0), xrs_reg = make_uint2(0, 0);
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    auto gload = [&](int64_t step) {
        const int64_t cw = step * tw * kNvRow, cx = step * tx * kNvRow;
#pragma unroll
        for (int i = 0; i < W_UNITS; i++)
            w_reg[i] = w_src[i] ? *reinterpret_cast<const uint4 *>(w_src[i] + cw) : zero4;
#pragma unroll
        for (int i = 0; i < X_UNITS; i++) {
            xb_reg[i] = xb_src[i] ? *reinterpret_cast<const uint4 *>(xb_src[i] + cx) : zero4;
            xr_reg[i] = xr_src[i] ? *reinterpret_cast<const uint4 *>(xr_src[i] + cx) : zero4;
        }
        const int64_t sw = step * tw * kNvScRow, sx = step * tx * kNvScRow;
        if (ws_src) ws_reg = *reinterpret_cast<const uint2 *>(ws_src + sw);
        if (xbs_src) xbs_reg = *reinterpret_cast<const uint2 *>(xbs_src + sx);
        if (xrs_src) xrs_reg = *reinterpret_cast<const uint2 *>(xrs_src + sx);
    };
    auto lstore = [&](uint8_t *st) {
#pragma unroll
        for (int i = 0; i < W_UNITS; i++) *reinterpret_cast<uint4 *>(st + L::W_CODES + w_lds[i]) = w_reg[i];
#pragma unroll
        for (int i = 0; i < X_UNITS; i++) {
            *reinterpret_cast<uint4 *>(st + L::XB_CODES + x_lds[i]) = xb_reg[i];
            *reinterpret_cast<uint4 *>(st + L::XR_CODES + x_lds[i]) = xr_reg[i];
        }
        if (BN >= NT || tid < BN) *reinterpret_cast<uint2 *>(st + L::W_SC + tid * kNvScRow) = ws_reg;
        if (BM >= NT || tid < BM) {
            *reinterpret_cast<uint2 *>(st + L::XB_SC + tid * kNvScRow) = xbs_reg;
            *reinterpret_cast<uint2 *>(st + L::XR_SC + tid * kNvScRow) = xrs_reg;
        }
    };

    v4f_nv acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = v4f_nv{0.0f, 0.0f, 0.0f, 0.0f};

    const int frow = lane & 15, fq = lane >> 4;
    const int64_t nsteps = K / kNvKS;
    gload(0);
    lstore(smem);
    __syncthreads();

    for (int64_t s = 0; s < nsteps; s++) {
        uint8_t *cur = smem + (s & 1) * L::BYTES;
        gload(s + 1 < nsteps ? s + 1 : s);  // see the MXFP4 kernel: one basic block per step
        __builtin_amdgcn_sched_barrier(0);

        v8bf wd[FN][4];
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = wn * (FN * 16) + j * 16 + frow;
            const uint4 c = *reinterpret_cast<const uint4 *>(cur + L::W_CODES + row * kNvRow + nv_swz(row, fq) * 16);
            const float s0 = e4m3_value(cur[L::W_SC + row * kNvScRow + 2 * fq]);
            const float s1 = e4m3_value(cur[L::W_SC + row * kNvScRow + 2 * fq + 1]);
            wd[j][0] = dequant8(c.x, s0);
            wd[j][1] = dequant8(c.y, s0);
            wd[j][2] = dequant8(c.z, s1);
            wd[j][3] = dequant8(c.w, s1);
        }
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wm * (FM * 16) + i * 16 + frow;
            const int off = row * kNvRow + nv_swz(row, fq) * 16;
            const uint4 cb = *reinterpret_cast<const uint4 *>(cur + L::XB_CODES + off);
            const uint4 cr = *reinterpret_cast<const uint4 *>(cur + L::XR_CODES + off);
            const float sb0 = e4m3_value(cur[L::XB_SC + row * kNvScRow + 2 * fq]);
            const float sb1 = e4m3_value(cur[L::XB_SC + row * kNvScRow + 2 * fq + 1]);
            const float sr0 = e4m3_value(cur[L::XR_SC + row * kNvScRow + 2 * fq]);
            const float sr1 = e4m3_value(cur[L::XR_SC + row * kNvScRow + 2 * fq + 1]);
            const uint32_t cbw[4] = {cb.x, cb.y, cb.z, cb.w};
            const uint32_t crw[4] = {cr.x, cr.y, cr.z, cr.w};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const v8bf xb = dequant8(cbw[t], t < 2 ? sb0 : sb1);
                const v8bf xr = dequant8(crw[t], t < 2 ? sr0 : sr1);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wd[j][t], xb, acc[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wd[j][t], xr, acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        lstore(smem + ((s + 1) & 1) * L::BYTES);
        __syncthreads();
    }

    const float alpha = __fmul_rn(*a.x_gscale, a.w_gscale[expert]);
#pragma unroll
    for (int i = 0; i < FM; i++) {
        const int64_t m = m0 + wm * (FM * 16) + i * 16 + frow;
        if (m >= m_end) continue;
        float *yrow = a.y + m * a.ldy;
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int64_t n = n0 + wn * (FN * 16) + j * 16 + fq * 4;
            const v4f_nv v = acc[i][j] * alpha;
            if (a.y_vec && n + 3 < a.nout) {
                *reinterpret_cast<v4f_nv *>(yrow + n) = v;
            } else {
                if (n < a.nout) yrow[n] = v.x;
                if (n + 1 < a.nout) yrow[n + 1] = v.y;
                if (n + 2 < a.nout) yrow[n + 2] = v.z;
                if (n + 3 < a.nout) yrow[n + 3] = v.w;
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_nv(const LinearArgs &a, hipStream_t st) {
    using L = NvStage<BM, BN>;
    const size_t lds = 2 * (size_t)L::BYTES;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_dual_gemm_nv<BM, BN, WM, WN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t mtiles = a.offsets ? (a.rows + BM - 1) / BM + a.E : (a.rows + BM - 1) / BM;
    const dim3 grid((unsigned)((a.nout + BN - 1) / BN), (unsigned)mtiles);
    hipLaunchKernelGGL((k_dual_gemm_nv<BM, BN, WM, WN>), grid, dim3(WM * WN * 64), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_linear(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st) {
    (void)ws;
    (void)ws_bytes;
    if (a.fmt == kFmtMx) return launch_linear_mx(a, st);
    if (a.rows <= 64 && !a.offsets) return launch_nv<64, 128, 2, 2>(a, st);
    return launch_nv<256, 128, 2, 2>(a, st);
}

size_t linear_workspace_bytes(int64_t rows, int64_t K, int64_t nout, int64_t E, int fmt) {
    (void)rows; (void)K; (void)nout; (void)E; (void)fmt;
    return 0;
}

}  // namespace sharq
