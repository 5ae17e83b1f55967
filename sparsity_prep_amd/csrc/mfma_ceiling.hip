// Stand-alone probe (not part of libsharq.so): throughput of back-to-back
// 32x32x64 block-scaled FP4 MFMAs issued from registers, the instruction the
// dual-path product runs on, with near-constant operands and with random
// E2M1 codes and E8M0 scales.  Each wave keeps 8 accumulators and feeds each
// one twice per 16 MFMAs, 4 instructions apart (the backbone / residual
// pattern of the product); 256 workgroups of 4 or 8 waves (1 or 2 per SIMD).
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o mfma_ceiling sparsity_prep_amd/csrc/mfma_ceiling.hip && ./mfma_ceiling
//
// Run it under `rocprofv3 --pmc GRBM_GUI_ACTIVE` to read the busy clock:
// cycles summed over the 8 XCDs / 8 / kernel time.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int OPSEL>
__device__ __forceinline__ v16f mfma(v4i a, v4i b, v16f c, int sa, int sb) {
    const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    const v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OPSEL, sa, OPSEL, sb);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_mfma_loop(float *out, const v4i *src, const int *scales, int iters) {
    const int lane = threadIdx.x & 63;
    v16f acc[8];
    v4i w[4], x[4];
    int sw[4], sx[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        w[j] = src[(lane + 64 * j) & 255];
        x[j] = src[(lane + 64 * j + 17) & 255];
        sw[j] = scales[(lane + 64 * j) & 255];
        sx[j] = scales[(lane + 64 * j + 29) & 255];
    }
#pragma unroll
    for (int j = 0; j < 8; j++)
        for (int q = 0; q < 16; q++) acc[j][q] = 0.0f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int t = 0; t < 2; t++) {
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int i = k / 8, p = (k / 4) & 1, j = k % 4;
                const int a = i * 4 + j, xi = 2 * i + p;
                if (t == 0)
                    acc[a] = mfma<0>(w[j], x[xi], acc[a], sw[j], sx[xi]);
                else
                    acc[a] = mfma<1>(w[j], x[xi], acc[a], sw[j], sx[xi]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++)
        for (int q = 0; q < 16; q++) s += acc[j][q];
    out[blockIdx.x * NW * 64 + threadIdx.x] = s;
}

#define CHECK(x)                                                              \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                         \
        }                                                                     \
    } while (0)

template <int NW>
static int run(const char *what, float *out, const v4i *src, const int *scales, int iters) {
    const int blocks = 256;
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(k_mfma_loop<NW>, dim3(blocks), dim3(NW * 64), 0, 0, out, src, scales, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e0, 0));
    for (int i = 0; i < 5; i++)
        hipLaunchKernelGGL(k_mfma_loop<NW>, dim3(blocks), dim3(NW * 64), 0, 0, out, src, scales, iters);
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= 5;
    const double flops = (double)blocks * NW * iters * 32 * 131072.0;
    printf("%-8s operands, %d waves/SIMD: %8.3f ms  %7.0f TFLOP/s\n", what, NW / 4, ms, flops / ms / 1e9);
    return 0;
}

int main() {
    float *out;
    v4i *src;
    int *scales;
    CHECK(hipMalloc(&out, 256 * 512 * sizeof(float)));
    CHECK(hipMalloc(&src, 256 * sizeof(v4i)));
    CHECK(hipMalloc(&scales, 256 * sizeof(int)));
    uint32_t codes[1024], sc[256];
    const int iters = 2000;
    for (int pass = 0; pass < 2; pass++) {
        uint32_t r = 12345u;
        for (int i = 0; i < 1024; i++) {  // xorshift32: random E2M1 nibbles, or one repeated byte
            r ^= r << 13;
            r ^= r >> 17;
            r ^= r << 5;
            codes[i] = pass ? r : 0x11111111u;
        }
        for (int i = 0; i < 256; i++)  // E8M0 scales near 2^0, random low bits per byte
            sc[i] = pass ? (0x7c7c7c7cu ^ (codes[i] & 0x03030303u)) : 0x7f7f7f7fu;
        CHECK(hipMemcpy(src, codes, sizeof(codes), hipMemcpyHostToDevice));
        CHECK(hipMemcpy(scales, sc, sizeof(sc), hipMemcpyHostToDevice));
        const char *what = pass ? "random" : "constant";
        if (run<4>(what, out, src, scales, iters) || run<8>(what, out, src, scales, iters)) return 1;
    }
    CHECK(hipFree(out));
    CHECK(hipFree(src));
    CHECK(hipFree(scales));
    return 0;
}
