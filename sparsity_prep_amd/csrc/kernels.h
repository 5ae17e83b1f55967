// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sharq {

enum { kNormNone = 0, kNormRms = 1, kNormLayer = 2 };
enum { kFmtMx = 0, kFmtNv = 1 };
// Product operand format: NVFP4 whose backbone is stored in the compressed
// form of the 2:4 sparse f16 matrix instruction (LinearArgs::fmt only; the
// preparation keeps fmt = kFmtNv and sets PrepArgs::sp).
constexpr int kFmtNvSp = 2;
// Bytes per row and K tile of the compressed backbone: 32 code bytes (two
// kept codes of every group of four) and 16 bytes of 2-bit positions.
constexpr int kSpRowBytes = 48;
enum { kOutF32 = 0, kOutBf16 = 1, kOutF16 = 2 };  // product output element type

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
    bool sp;     // NVFP4 backbone in the 2:4 compressed form (needs off32 and 2:4)
    // SiLU(gate)*up source (sharq_prepare_swiglu): rows of gu with stride ldgu
    // floats, gate in [0, K), up in [K, 2K); x is unused then
    const float *gu;
    int64_t ldgu;
};

hipError_t launch_prepare(const PrepArgs &a, void *ws, hipStream_t st);
// The same preparation with its scratch (NVFP4 per-row statistics, at most
// kNoallocRows rows) in the library's own device array: allocates nothing.
constexpr int64_t kNoallocRows = 65536;
hipError_t launch_prepare_noalloc(const PrepArgs &a, hipStream_t st);
hipError_t launch_prepare_swiglu(const PrepArgs &a, void *ws, hipStream_t st);
size_t prepare_workspace_bytes(int64_t T, int fmt);

struct QuantWArgs {
    const uint16_t *w;
    int64_t E, nout, K, ldw;  // element k of row n of expert e at w[(e*nout + n)*ldw + k]
    int fmt;
    bool bf16;
    uint8_t *codes, *scales;
    float *global_scale;
    // gate/up weight (gate rows [0, nout/2), up rows [nout/2, nout)) stored
    // with the two halves interleaved in 32-row groups: payload row
    // 64p + c holds gate row 32p + c, row 64p + 32 + c up row 32p + c
    bool gate_up_interleave;
};

// Payload row of source row n of a gate/up weight of nout rows, interleaved
// as above.
__host__ __device__ inline int64_t gate_up_row(int64_t n, int64_t nout) {
    const int64_t h = nout / 2, up = n >= h ? 1 : 0, r = n - up * h;
    return (r / 32) * 64 + up * 32 + r % 32;
}

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
    void *y;     // [rows][ldy] elements of type ydt
    int ydt;     // kOutF32, kOutBf16 or kOutF16 (rounded to nearest even)
    int64_t ldy;
    bool y_vec;  // y and its rows aligned to four elements: one vector store per four
    // K split (dense products only): grid row s multiplies K tiles
    // [s*ksplit_tiles, (s+1)*ksplit_tiles) into y + s*split_stride; 0 = no split
    int64_t ksplit_tiles, split_stride;
    // dense tile order: 0 = each XCD takes a run of column tiles (all row
    // tiles of each), RB > 0 = each XCD takes a band of RB row tiles and a
    // share of the column tiles (set by the launcher)
    int64_t xcd_band;
    // SwiGLU epilogue (launch_linear_swiglu, MXFP4): the weight rows are a
    // gate/up pair interleaved in 32-row groups (gate_up_row); the product's
    // FP32 rows become the next linear's prepared MXFP4 activation of rows x
    // nout/2 elements, x = SiLU(gate) * up with an N:M mask (M in {1, 2, 4});
    // y (FP32, may be null) additionally receives the product itself
    uint8_t *p_mask, *p_b_codes, *p_b_scales, *p_r_codes, *p_r_scales;
    int p_n, p_m;
};

hipError_t launch_linear(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_linear_swiglu(const LinearArgs &a, hipStream_t st);
size_t linear_workspace_bytes(int64_t rows, int64_t K, int64_t nout, int64_t E, int fmt);

}  // namespace sharq
