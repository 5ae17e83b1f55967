// Weight quantization for gfx950: the single FP4 weight payload that both
// SharQ paths read (SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract: one payload,
// a scale view per path).  Round-to-nearest-even into
// MXFP4 (E8M0 per 32) or NVFP4 (E4M3 per 16 times one FP32 scale per expert).
// Run once per weight; the lane layout matches the prep kernel (eight
// consecutive elements per lane, 128-bit loads).
#include "device_util.h"
#include "kernels.h"

namespace sharq {

constexpr int kQWaves = 4;
constexpr int kQChunk = 512;
constexpr int kQChunks = 4;  // chunks per wave task

template <int FMT>
__device__ __forceinline__ uint32_t quant_block8(const float v[8], float G, float G6, uint32_t &codes) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, dpp_f32<kDppQuadXor1>(m));
    uint32_t c = 0, sb;
    if constexpr (FMT == kFmtMx) {
        m = fmaxf(m, dpp_f32<kDppQuadXor2>(m));
        const int E = mx_shared_exp(m);
        const float inv = pow2_neg(E);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float q;
            c |= e2m1_encode(__fmul_rn(v[i], inv), q) << (4 * i);
        }
        sb = (uint32_t)(E + 127);
    } else {
        sb = e4m3_encode_sat(__fdiv_rn(m, G6));
        const float D = __fmul_rn(e4m3_value(sb), G);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float q;
            if (sb != 0u) c |= e2m1_encode(__fdiv_rn(v[i], D), q) << (4 * i);
        }
    }
    codes = c;
    return sb;
}

// Task = (row of [E*nout], kQChunks chunks).
template <bool BF16, int FMT>
__global__ __launch_bounds__(kQWaves * kWave) void k_quant_w(QuantWArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t K = a.K;
    const int64_t tpr = (K + (int64_t)kQChunk * kQChunks - 1) / ((int64_t)kQChunk * kQChunks);
    const int64_t task = (int64_t)blockIdx.x * kQWaves + (threadIdx.x >> 6);
    const int64_t row = task / tpr;
    if (row >= a.E * a.nout) return;
    const int64_t c0 = (task - row * tpr) * kQChunks;
    float G = 1.0f, G6 = 6.0f;
    if constexpr (FMT == kFmtNv) {
        G = a.global_scale[row / a.nout];
        G6 = __fmul_rn(6.0f, G);
    }
    constexpr int B = FMT == kFmtMx ? 32 : 16;
    constexpr int LPB = B / 8;
#pragma unroll
    for (int c = 0; c < kQChunks; c++) {
        const int64_t e0 = ((c0 + c) * kWave + lane) * 8;
        if (e0 < K) {
            float v[8];
            unpack8<BF16>(*reinterpret_cast<const uint4 *>(a.w + row * a.ldw + e0), v);
            uint32_t codes;
            const uint32_t sb = quant_block8<FMT>(v, G, G6, codes);
            // expert-major; each expert's [nout x K] payload is K-tiled
            const int64_t ex = row / a.nout, ns = row - ex * a.nout;
            const int64_t n = a.gate_up_interleave ? gate_up_row(ns, a.nout) : ns;
            *reinterpret_cast<uint32_t *>(a.codes + ex * a.nout * (K / 2) + ktile_offset<2>(n, e0, a.nout, K)) = codes;
            if ((lane % LPB) == 0) a.scales[ex * a.nout * (K / B) + ktile_offset<B>(n, e0, a.nout, K)] = (uint8_t)sb;
        }
    }
}

// NVFP4: per-row amax, then per-expert tensor scale.
template <bool BF16>
__global__ __launch_bounds__(kQWaves * kWave) void k_row_amax(QuantWArgs a, float *row_amax) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kQWaves + (threadIdx.x >> 6);
    if (row >= a.E * a.nout) return;
    float m = 0.0f, v[8];
    for (int64_t e0 = (int64_t)lane * 8; e0 < a.K; e0 += kQChunk) {
        unpack8<BF16>(*reinterpret_cast<const uint4 *>(a.w + row * a.ldw + e0), v);
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) row_amax[row] = m;
}

__global__ __launch_bounds__(256) void k_expert_scale(const float *row_amax, int64_t nout, float *G) {
    __shared__ float part[256 / kWave];
    const int64_t e = blockIdx.x;
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < nout; i += blockDim.x) m = fmaxf(m, row_amax[e * nout + i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
        const float g = __fdiv_rn(t, 2688.0f);
        G[e] = g > 0.0f ? g : 1.0f;
    }
}

__global__ void k_fill_ones(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 1.0f;
}

template <bool BF16, int FMT>
static hipError_t launch_qw(const QuantWArgs &a, void *ws, hipStream_t st) {
    const int64_t rows = a.E * a.nout;
    if constexpr (FMT == kFmtNv) {
        float *row_amax = reinterpret_cast<float *>(ws);
        hipLaunchKernelGGL((k_row_amax<BF16>), dim3((unsigned)((rows + kQWaves - 1) / kQWaves)),
                           dim3(kQWaves * kWave), 0, st, a, row_amax);
        hipLaunchKernelGGL(k_expert_scale, dim3((unsigned)a.E), dim3(256), 0, st, row_amax, a.nout,
                           a.global_scale);
    } else if (a.global_scale) {
        hipLaunchKernelGGL(k_fill_ones, dim3((unsigned)((a.E + 255) / 256)), dim3(256), 0, st,
                           a.global_scale, a.E);
    }
    const int64_t tpr = (a.K + (int64_t)kQChunk * kQChunks - 1) / ((int64_t)kQChunk * kQChunks);
    const int64_t tasks = rows * tpr;
    hipLaunchKernelGGL((k_quant_w<BF16, FMT>), dim3((unsigned)((tasks + kQWaves - 1) / kQWaves)),
                       dim3(kQWaves * kWave), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_quantize_weight(const QuantWArgs &a, void *ws, hipStream_t st) {
    if (a.E * a.nout == 0) return hipSuccess;
    if (a.bf16) return a.fmt == kFmtMx ? launch_qw<true, kFmtMx>(a, ws, st) : launch_qw<true, kFmtNv>(a, ws, st);
    return a.fmt == kFmtMx ? launch_qw<false, kFmtMx>(a, ws, st) : launch_qw<false, kFmtNv>(a, ws, st);
}

size_t quantize_weight_workspace_bytes(int64_t E, int64_t nout, int fmt) {
    return fmt == kFmtNv ? (size_t)(E * nout > 0 ? E * nout : 1) * sizeof(float) : 0;
}

}  // namespace sharq
