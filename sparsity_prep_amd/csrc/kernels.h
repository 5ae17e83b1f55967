// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sharq {

enum { kNormNone = 0, kNormRms = 1, kNormLayer = 2 };
enum { kFmtMx = 0, kFmtNv = 1 };

// K-tiled layout of every FP4 code and scale array (activations and
// weights): K is cut into tiles of 128 elements (the last one may be
// shorter); tile t stores all `rows` rows back to back, each row holding the
// tile's codes (w/2 bytes for a tile of width w) or scales (w/B bytes).  One
// K step of the products thus reads one contiguous run per array instead of
// a short piece of every row.  `per` is elements per byte: 2 for codes, the
// block size B for scales; K is a multiple of B.
constexpr int kTileK = 128;

template <int PER>
__host__ __device__ inline int64_t ktile_offset(int64_t row, int64_t e, int64_t rows, int64_t K) {
    static_assert(PER == 2 || PER == 16 || PER == 32, "codes or block scales");
    const uint64_t t = (uint64_t)e / kTileK;
    const uint64_t rem = (uint64_t)K - t * kTileK;
    const uint64_t w = rem < (uint64_t)kTileK ? rem : (uint64_t)kTileK;
    return (int64_t)(t * (uint64_t)rows * (kTileK / PER) + (uint64_t)row * (w / PER) +
                     ((uint64_t)e % kTileK) / PER);
}

struct PrepArgs {
    const uint16_t *x;
    int64_t T, K, ldx;
    const uint16_t *gamma, *beta;
    float eps;
    int n, m, norm, fmt;
    bool bf16;
    uint8_t *mask, *b_codes, *b_scales, *r_codes, *r_scales;
    float *global_scale;
    bool off32;  // K % 128 == 0 and T*K/2 < 2^32: 32-bit K-tiled offsets
    // SiLU(gate)*up source (sharq_prepare_swiglu): rows of gu with stride ldgu
    // floats, gate in [0, K), up in [K, 2K); x is unused then
    const float *gu;
    int64_t ldgu;
};

hipError_t launch_prepare(const PrepArgs &a, void *ws, hipStream_t st);
hipError_t launch_prepare_swiglu(const PrepArgs &a, void *ws, hipStream_t st);
size_t prepare_workspace_bytes(int64_t T, int fmt);

struct QuantWArgs {
    const uint16_t *w;
    int64_t E, nout, K;
    int fmt;
    bool bf16;
    uint8_t *codes, *scales;
    float *global_scale;
};

hipError_t launch_quantize_weight(const QuantWArgs &a, void *ws, hipStream_t st);
size_t quantize_weight_workspace_bytes(int64_t E, int64_t nout, int fmt);

struct LinearArgs {
    const uint8_t *b_codes, *b_scales, *r_codes, *r_scales;
    const float *x_gscale;
    int64_t T, K;
    int fmt;
    const uint8_t *w_codes, *w_scales;
    const float *w_gscale;
    int64_t E, nout;
    const int32_t *offsets, *row_index;
    int64_t rows;
    float *y;
    int64_t ldy;
    bool y_vec;  // rows of y are 16-byte aligned: 128-bit stores
    // K split (dense products only): grid row s multiplies K tiles
    // [s*ksplit_tiles, (s+1)*ksplit_tiles) into y + s*split_stride; 0 = no split
    int64_t ksplit_tiles, split_stride;
};

hipError_t launch_linear(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st);
size_t linear_workspace_bytes(int64_t rows, int64_t K, int64_t nout, int64_t E, int fmt);

}  // namespace sharq
