// Test support (not part of the library): the gfx950 2:4 sparse f16 matrix
// instruction v_smfmac_f32_32x32x32_f16, run on caller data so that a test
// can check its operand layout against a host model, and two throughput
// loops (the sparse instruction and the dense v_mfma_f32_32x32x16_f16 that
// covers half its K) for the comparison of their rates.  One wave of 64
// lanes: lane l passes A[l] (8 halves: the kept values of its sparse row
// segment), B[l] (16 halves), the index word idx[l] and receives D[l] (16
// floats).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v16h __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int ABID>
__global__ __launch_bounds__(64) void k_smfmac_once(const v8h *a, const v16h *b, const int *idx, v16f *d) {
    const int l = threadIdx.x;
    v16f acc = {};
    acc = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a[l], b[l], acc, idx[l], 0, ABID);
    d[l] = acc;
}

// Four independent accumulator chains per wave; the sum of the accumulators
// is written so that no instruction is dead.
__global__ __launch_bounds__(256) void k_rate_sparse(const v8h *a, const v16h *b, float *out, int iters) {
    const int l = threadIdx.x & 63;
    const v8h x = a[l];
    const v16h y = b[l];
    v16f acc[4] = {};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++) acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(x, y, acc[j], 0x44444444, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_rate_dense(const v8h *a, float *out, int iters) {
    const int l = threadIdx.x & 63;
    const v8h x = a[l];
    v16f acc[4] = {};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, x, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// D = smfmac(A, B, 0, idx) with index half `abid` (0: bits 0-15 of the
// index word, 1: bits 16-31); device buffers of 64*8 and 64*16 halves, 64
// ints, 64*16 floats.  Returns the HIP error code.
extern "C" __attribute__((visibility("default"))) int probe_smfmac(const void *a, const void *b, const int *idx,
                                                                    float *d, int abid, void *stream) {
    if (!a || !b || !idx || !d || (abid != 0 && abid != 1)) return (int)hipErrorInvalidValue;
    if (abid == 0)
        hipLaunchKernelGGL(k_smfmac_once<0>, dim3(1), dim3(64), 0, (hipStream_t)stream, (const v8h *)a,
                           (const v16h *)b, idx, (v16f *)d);
    else
        hipLaunchKernelGGL(k_smfmac_once<1>, dim3(1), dim3(64), 0, (hipStream_t)stream, (const v8h *)a,
                           (const v16h *)b, idx, (v16f *)d);
    return (int)hipGetLastError();
}

// Throughput loop: sparse != 0 runs the sparse instruction, else the dense
// one; `blocks` workgroups of four waves, `iters` iterations of four
// instructions per wave; out holds blocks*256 floats, a and b the operands
// of probe_smfmac.  Returns the HIP error code.
extern "C" __attribute__((visibility("default"))) int probe_rate(int sparse, const void *a, const void *b,
                                                                  float *out, int blocks, int iters, void *stream) {
    if (!a || !b || !out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    if (sparse)
        hipLaunchKernelGGL(k_rate_sparse, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const v8h *)a,
                           (const v16h *)b, out, iters);
    else
        hipLaunchKernelGGL(k_rate_dense, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const v8h *)a, out,
                           iters);
    return (int)hipGetLastError();
}
