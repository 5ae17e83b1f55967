// Test support (not part of the library): runs the library's own device
// encoders over a range of float32 bit patterns, one result per output
// byte, so that a test can compare every float32 input with the oracle:
// the E2M1 conversion (sharq::e2m1_cvt8: the hardware FP32 -> FP4
// conversion with scale 1 plus the canonical-zero fix), the E4M3 block-scale
// encoder (sharq::e4m3_encode_sat), the MX shared exponent
// (sharq::mx_shared_exp, written as the E8M0 byte E + 127), and SiLU(g)
// (sharq::silu_times_n and sharq::silu_times_inrange with u = 1, which
// returns the quotient itself), and the NVFP4 element quotient
// float(double(x) * sharq::rcp_f64_refined(d)).
#include "../../sparsity_prep_amd/csrc/device_util.h"

__global__ void k_probe_e2m1(uint32_t base, uint32_t n, uint8_t *out) {
    const uint32_t i = (blockIdx.x * blockDim.x + threadIdx.x) * 8u;
    if (i >= n) return;
    float u[8];
#pragma unroll
    for (int k = 0; k < 8; k++) u[k] = __uint_as_float(base + i + (uint32_t)k);
    const uint32_t p = sharq::e2m1_cvt8(u, 1.0f);
#pragma unroll
    for (int k = 0; k < 8; k++) out[i + k] = (uint8_t)((p >> (4 * k)) & 0xFu);
}

__global__ void k_probe_scales(uint32_t base, uint32_t n, uint8_t *e4m3, uint8_t *e8m0) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float t = __uint_as_float(base + i);
    e4m3[i] = (uint8_t)sharq::e4m3_encode_sat(t);
    e8m0[i] = (uint8_t)(sharq::mx_shared_exp(t) + 127);
}

// Codes of the n patterns base .. base + n - 1 (n a multiple of 8, at most
// 2^31, base + n <= 2^32) into out[0 .. n); returns the HIP error code.
extern "C" __attribute__((visibility("default"))) int probe_e2m1(uint32_t base, uint32_t n, uint8_t *out,
                                                                  void *stream) {
    if (n % 8u != 0u || n > (1u << 31) || (uint64_t)base + n > (1ull << 32) || out == nullptr)
        return (int)hipErrorInvalidValue;
    const uint32_t threads = n / 8u, block = 256u;
    hipLaunchKernelGGL(k_probe_e2m1, dim3((threads + block - 1) / block), dim3(block), 0,
                       (hipStream_t)stream, base, n, out);
    return (int)hipGetLastError();
}

// E4M3 bytes and E8M0 bytes of the n patterns base .. base + n - 1 (same
// limits as probe_e2m1; the patterns should be non-negative finite floats,
// the encoders' domain).
extern "C" __attribute__((visibility("default"))) int probe_scales(uint32_t base, uint32_t n, uint8_t *e4m3,
                                                                    uint8_t *e8m0, void *stream) {
    if (n > (1u << 31) || (uint64_t)base + n > (1ull << 32) || e4m3 == nullptr || e8m0 == nullptr)
        return (int)hipErrorInvalidValue;
    const uint32_t block = 256u;
    hipLaunchKernelGGL(k_probe_scales, dim3((n + block - 1) / block), dim3(block), 0, (hipStream_t)stream, base,
                       n, e4m3, e8m0);
    return (int)hipGetLastError();
}

// SiLU of every pattern: mode 0 through silu_times_n<8> (eight consecutive
// patterns per lane, so a wave takes the short form exactly when all of its
// 512 patterns lie in [-80, 80]); mode 1 through silu_times_inrange wherever
// |g| <= 80 (silu_times elsewhere).
__global__ void k_probe_silu(uint32_t base, uint32_t n, int mode, float *out) {
    const uint32_t i = (blockIdx.x * blockDim.x + threadIdx.x) * 8u;
    if (i >= n) return;
    float g[8], one[8], h[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        g[k] = __uint_as_float(base + i + (uint32_t)k);
        one[k] = 1.0f;
    }
    if (mode == 0) {
        sharq::silu_times_n<8>(g, one, h);
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++)
            h[k] = fabsf(g[k]) <= 80.0f ? sharq::silu_times_inrange(g[k], 1.0f) : sharq::silu_times(g[k], 1.0f);
    }
#pragma unroll
    for (int k = 0; k < 8; k++) out[i + k] = h[k];
}

// SiLU values of the n patterns base .. base + n - 1 into out[0 .. n) (same
// limits as probe_e2m1; mode 0 or 1 as in k_probe_silu).
extern "C" __attribute__((visibility("default"))) int probe_silu(uint32_t base, uint32_t n, int mode, float *out,
                                                                  void *stream) {
    if (n % 8u != 0u || n > (1u << 31) || (uint64_t)base + n > (1ull << 32) || out == nullptr ||
        (mode != 0 && mode != 1))
        return (int)hipErrorInvalidValue;
    const uint32_t threads = n / 8u, block = 256u;
    hipLaunchKernelGGL(k_probe_silu, dim3((threads + block - 1) / block), dim3(block), 0, (hipStream_t)stream, base,
                       n, mode, out);
    return (int)hipGetLastError();
}

// NVFP4 element quotients q[i] = float(double(x[i]) * rcp_f64_refined(d[i]))
// as the prep kernels form them (d[i] positive finite floats).
__global__ void k_probe_quotient(const float *x, const float *d, uint32_t n, float *q) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    q[i] = (float)((double)x[i] * sharq::rcp_f64_refined((double)d[i]));
}

// Quotients of the n pairs (x[i], d[i]) into q[0 .. n) (n at most 2^31);
// returns the HIP error code.
extern "C" __attribute__((visibility("default"))) int probe_quotient(const float *x, const float *d, uint32_t n,
                                                                      float *q, void *stream) {
    if (n > (1u << 31) || x == nullptr || d == nullptr || q == nullptr) return (int)hipErrorInvalidValue;
    const uint32_t block = 256u;
    hipLaunchKernelGGL(k_probe_quotient, dim3((n + block - 1) / block), dim3(block), 0, (hipStream_t)stream, x, d,
                       n, q);
    return (int)hipGetLastError();
}
