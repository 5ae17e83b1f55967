// Dual-path FP4 linear layer for gfx950 (MXFP4 and NVFP4) and its dispatcher.
//
// Source: SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference, Abstract.  The backbone product (sparse path) and the residual
// product (dense path, which restores what masking dropped and what backbone
// rounding lost) read one FP4 weight payload.
//
// Y[m][n] = sum_k (Qb[m][k] + Qr[m][k]) * W[n][k], evaluated as two matrix
// products into one FP32 accumulator: every weight fragment is read from LDS
// once and feeds the backbone MFMA and the residual MFMA.  MXFP4 multiplies
// the backbone densely on its zero-filled form: gfx950's sparse matrix
// instructions (smfmac) take fp8, bf8, f16, bf16 or int8 operands without
// block scales, so none holds MXFP4.  NVFP4, which is multiplied as exactly
// dequantized f16 values, can feed its backbone to the 2:4 sparse f16
// instruction when the preparation stored it in that instruction's
// compressed form (NVFP4_SP24).
//
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and per-lane
//          E8M0 scales (16x16x128 in the small-T kernel).
//   NVFP4: an E2M1 code times an E4M3 scale needs up to 6 significant bits,
//          which no FP4/FP6/FP8 operand holds and a power-of-two block scale
//          cannot express; f16 holds it exactly (as does bf16, but gfx950
//          multiplies packed f16 and not packed bf16).  The fragments are
//          dequantized in registers (hardware FP4 -> f16 conversion with the
//          scale's power of two, one packed f16 multiply by its mantissa)
//          and multiplied with v_mfma_f32_32x32x16_f16; the two tensor
//          scales (activation and weight) are applied to the FP32
//          accumulator in the epilogue.
//
// Operand mapping: the weight fragment is the A operand, the activation
// fragment the B operand, so every group of four accumulator values is four
// consecutive output columns of one token row and leaves as one 128-bit
// store.  Each lane feeds 16 bytes of codes (32 elements of one row).
#include <type_traits>

#include "device_util.h"
#include "kernels.h"

namespace sharq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v16h __attribute__((ext_vector_type(16)));

constexpr int kCbszFp4 = 4;  // MFMA operand format code for E2M1

// 32x32x64 block-scaled FP4 MFMA: lane l feeds row l%32 and the 32-element
// block l/32 of the 64-wide K step; lane l, accumulator r holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].  On gfx950 this shape runs FP4 at twice
// the FP8 rate (8.8 PFLOP/s measured with constant operands, 6.3 with random
// ones, at which the chip lowers its clock), the 16x16x128 shape does not.
// OPSEL picks which byte of the scale registers this MFMA uses.
template <int OPSEL>
__device__ __forceinline__ v16f mfma32_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
    const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    const v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kCbszFp4, kCbszFp4, OPSEL, sa, OPSEL, sb);
}

// 16x16x128 block-scaled FP4 MFMA (lane l: row l%16, block l/16).
template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_sel(v4i a, v4i b, v4f c, int sa, int sb) {
    const v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    const v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, kCbszFp4, kCbszFp4, OPSEL, sa,
                                                           OPSEL, sb);
}

// NVFP4 fragment dequantization.  A lane's fragment is 32 E2M1 codes (16
// bytes, element e in nibble e) whose two 16-element halves carry E4M3
// scales in bytes 0 and 1 of its scale pair.  A scale s = 2^e * mant is
// applied as the hardware conversion's power of two (FP4 -> f16 pairs)
// followed by a packed f16 multiply by mant; code * s has at most 6
// significant bits and a magnitude in [2^-10, 2880] (or is 0), so every step
// is exact in f16.  The scale pair is decoded once (the hardware FP8, OCP
// E4M3, conversion is exact, subnormal scales included): the power of two of
// each half and both f16 mantissas in one register; then group t (elements
// 8t..8t+7, half t/2) is converted on demand.
typedef float v2f __attribute__((ext_vector_type(2)));

struct NvScale {
    float p2[2];
    v2h mp;
};

__device__ __forceinline__ NvScale nv_scale(uint32_t sc2) {
    const v2f sv = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc2, false);
    NvScale o;
    const uint32_t b0 = __float_as_uint(sv.x), b1 = __float_as_uint(sv.y);
    o.p2[0] = __uint_as_float(b0 & 0xFF800000u);
    o.p2[1] = __uint_as_float(b1 & 0xFF800000u);
    o.mp = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_pkrtz(__uint_as_float((b0 & 0x007FFFFFu) | 0x3F800000u),
                                                               __uint_as_float((b1 & 0x007FFFFFu) | 0x3F800000u)));
    return o;
}

template <int t>
__device__ __forceinline__ v8h nv_group(v4i c, const NvScale &s) {
    const uint32_t word = (uint32_t)c[t];
    const _Float16 m = s.mp[t / 2];
    const v2h mm = {m, m};
    const v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, s.p2[t / 2], 0) * mm;
    const v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, s.p2[t / 2], 1) * mm;
    const v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, s.p2[t / 2], 2) * mm;
    const v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, s.p2[t / 2], 3) * mm;
    return v8h{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
}

// 2:4 compressed backbone (NVFP4_SP24): the eight kept codes of one
// 16-element half u of the lane's sub-step, one code dword; codes 0-3 come
// from block u of unit T (scale pair `lo`), codes 4-7 from block u of unit
// 2+T (scale pair `hi`), exact in f16 as above.
template <int u>
__device__ __forceinline__ v8h sp_group(uint32_t word, const NvScale &lo, const NvScale &hi) {
    const v2h ml = {lo.mp[u], lo.mp[u]}, mh = {hi.mp[u], hi.mp[u]};
    const v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, lo.p2[u], 0) * ml;
    const v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, lo.p2[u], 1) * ml;
    const v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, hi.p2[u], 2) * mh;
    const v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, hi.p2[u], 3) * mh;
    return v8h{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
}

// gfx950 2:4 sparse f16 MFMA, D = A * B + D: A (tokens) holds the eight kept
// values of K 16h..16h+15 of its row (h = lane / 32), two per group of four
// at the 2-bit positions in bits 16u.. of `idx` (index half u = ABID); B
// (weights) holds K 8h..8h+7 in halves 0-7 and K 16+8h..16+8h+7 in halves
// 8-15.  Written as inline assembly with the accumulator in the
// accumulation registers: the compiler's builtin moved every accumulator of
// a 256x256 tile out of and back into them around each instruction.  The
// compiler does not know this is a matrix instruction, so the caller keeps
// other matrix instructions on the same accumulator at a distance (see the
// NVFP4_SP24 branch of DualGemm::mma); every accumulator's last writer is a
// compiler-visible MFMA (a residual product), so the epilogue's reads are
// spaced by the compiler.  Nor does it space the vector instructions that
// produce the operands from the matrix instruction that reads them: PAD puts
// two wait states in front (the first instruction of a group).
template <int ABID, bool PAD = false>
__device__ __forceinline__ void smfmac32_f16(v16f &acc, v8h a, v16h b, uint32_t idx) {
    if constexpr (PAD && ABID == 0)
        asm volatile("s_nop 1\n\tv_smfmac_f32_32x32x32_f16 %0, %1, %2, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
    else if constexpr (PAD)
        asm volatile("s_nop 1\n\tv_smfmac_f32_32x32x32_f16 %0, %1, %2, %3 abid:1" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
    else if constexpr (ABID == 0)
        asm volatile("v_smfmac_f32_32x32x32_f16 %0, %1, %2, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
    else
        asm volatile("v_smfmac_f32_32x32x32_f16 %0, %1, %2, %3 abid:1" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
}

// Output element conversions, round to nearest even (the hardware
// conversions; F16 overflows to infinity).
__device__ __forceinline__ uint32_t out_bits16(float f, int ydt) {
    return ydt == kOutBf16 ? (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f)
                           : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// One output Y[m][n] in the output type.
__device__ __forceinline__ void store_out1(const LinearArgs &a, int64_t m, int64_t n, float v) {
    if (a.ydt == kOutF32)
        static_cast<float *>(a.y)[m * a.ldy + n] = v;
    else
        static_cast<uint16_t *>(a.y)[m * a.ldy + n] = (uint16_t)out_bits16(v, a.ydt);
}

// Four consecutive outputs Y[m][n..n+3] (columns >= nout are skipped) in the
// output type: one vector store when the row allows it.
__device__ __forceinline__ void store_out4(const LinearArgs &a, int64_t m, int64_t n, v4f v) {
    if (a.ydt == kOutF32) {
        float *yrow = static_cast<float *>(a.y) + m * a.ldy;
        if (a.y_vec && n + 3 < a.nout) {
            *reinterpret_cast<v4f *>(yrow + n) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (n + i < a.nout) yrow[n + i] = v[i];
        }
    } else {
        uint16_t *yrow = static_cast<uint16_t *>(a.y) + m * a.ldy;
        const uint32_t h0 = out_bits16(v.x, a.ydt), h1 = out_bits16(v.y, a.ydt);
        const uint32_t h2 = out_bits16(v.z, a.ydt), h3 = out_bits16(v.w, a.ydt);
        if (a.y_vec && n + 3 < a.nout) {
            *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        } else {
            const uint32_t h[4] = {h0, h1, h2, h3};
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (n + i < a.nout) yrow[n + i] = (uint16_t)h[i];
        }
    }
}

// ============================================================================
// Prefill: LDS-tiled pipeline (three stage buffers in the shapes used; two
// supported) fed by direct global->LDS buffer loads (no register staging).
// Block tile BM token rows x BN weight rows, WGM x WGN waves, K stage 128 =
// two 64-wide sub-steps.
//
// A stage is one K tile of the K-tiled operand layout, so each array's stage
// is one contiguous run of rows x 64 code bytes (rows x SB scale bytes,
// SB = 4 for MXFP4, 8 for NVFP4) in HBM.  LDS row = four 16-byte units; unit
// u of row r sits at u ^ ((r >> 2) & 3) so that the rows one MFMA operand
// fetch reads spread over all banks.  A direct load writes 64 consecutive
// slots (one per lane), so each lane fetches whichever global bytes belong
// in its slot.
//
// Step s (stage s in buffer s % 3), every wave:
//   1. MFMAs of sub-step 0 (fragments read during step s-1), with the LDS
//      reads of stage s's sub-step-1 fragments and the last LSPLIT direct
//      loads of stage s+2 (into buffer (s+2) % 3, free since step s-1's
//      barrier) threaded between them;
//   2. wait until its own LDS reads are done and its own loads of stage s+1
//      have landed, then barrier: every wave is past its reads of stage s
//      and all of stage s+1 is in LDS;
//   3. MFMAs of sub-step 1, with the other direct loads of stage s+3 into
//      buffer s % 3 and the LDS reads of stage s+1's scales and sub-step-0
//      fragments threaded between them (RPS reads per MFMA).
// A stage's global loads thus have 1.5 to 2 steps to land, every LDS read
// has the rest of a sub-step to complete, and no wave holds its matrix unit
// idle behind a burst of memory instructions.  The buffers are distinct LDS
// variables so that the compiler's own wait before an LDS read only covers
// the loads into that buffer.  With two stages (NS = 2) the loads of stage
// s+2 all go into buffer s % 2 in step s and have one step to land.
//
// In sub-step T lane l feeds row l%32 of its fragment and the 32 elements of
// unit 2q + T, q = l/32 (both operands use the same unit, so the two
// sub-steps cover the stage's 128 elements).
// ============================================================================
constexpr int kKS = 128;            // K elements per stage
constexpr int kRowBytes = kKS / 2;  // 64 B of codes per row per stage

template <int FMT, int BM, int BN, int NW>
struct StageLayout {
    static constexpr int SB = FMT == kFmtMx ? 4 : 8;  // scale bytes per row per stage
    static constexpr int W_CODES = 0;
    static constexpr int XB_CODES = W_CODES + BN * kRowBytes;
    static constexpr int XR_CODES = XB_CODES + BM * kRowBytes;
    static constexpr int W_SC = XR_CODES + BM * kRowBytes;
    static constexpr int XB_SC = W_SC + BN * SB;
    static constexpr int XR_SC = XB_SC + BM * SB;
    static constexpr int BYTES = XR_SC + BM * SB;
    // direct-load instructions per wave per stage: 16-byte code slots, 16
    // rows per instruction; 4-byte scale slots, RPI rows per instruction,
    // spread over the waves (surplus waves repeat an earlier instruction:
    // identical bytes to identical places)
    static constexpr int W_NI = BN / 16, X_NI = BM / 16;  // 16-row code loads per array
    static constexpr int W_LD = (W_NI + NW - 1) / NW;
    static constexpr int X_LD = (X_NI + NW - 1) / NW;
    static constexpr int RPI = 64 * 4 / SB;
    static constexpr int SC_W = BN / RPI, SC_X = BM / RPI, SC_TOT = SC_W + 2 * SC_X;
    static constexpr int SC_LD = (SC_TOT + NW - 1) / NW;
    static constexpr int PER_STAGE = W_LD + 2 * X_LD + SC_LD;
    static_assert(BN % 16 == 0 && BM % 16 == 0, "tile rows per load");
    static_assert(BN % RPI == 0 && BM % RPI == 0, "scale rows per instruction");
};

// LDS stage buffers, sized per tile shape (so smaller tiles leave room for
// a second workgroup on the CU); an unused third buffer is never referenced
// and takes no LDS.
constexpr int kLdsBytes = 160 * 1024;
template <int BYTES> __shared__ __align__(16) uint8_t g_stage0[BYTES];
template <int BYTES> __shared__ __align__(16) uint8_t g_stage1[BYTES];
template <int BYTES> __shared__ __align__(16) uint8_t g_stage2[BYTES];

template <int B, int BYTES>
__device__ __forceinline__ uint8_t *stage_buf() {
    return B == 0 ? g_stage0<BYTES> : (B == 1 ? g_stage1<BYTES> : g_stage2<BYTES>);
}

__device__ __forceinline__ int swz_unit(int row, int unit) { return unit ^ ((row >> 2) & 3); }

// s_waitcnt on the vector-memory counter (at most N outstanding) and, with
// LGKM0, on the LDS counter (none outstanding); gfx9 encoding.
template <int N, bool LGKM0 = false>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8));
}

struct TileRows {
    int64_t m0;      // first output row of the tile
    int64_t m_end;   // one past the last valid output row
    int64_t expert;
};

// Grouped tiles: the tiles of expert e cover rows offsets[e]..offsets[e+1]-1
// in BM-row steps.
template <int BM>
__device__ __forceinline__ bool grouped_tile_rows(const LinearArgs &a, int64_t tile, TileRows &tr) {
    // Every wave finds the expert whose tile range holds `tile` on its own:
    // lane l takes expert base + l, the wave's inclusive prefix sum of the
    // experts' tile counts places each range, and one ballot picks the
    // lane whose range contains the tile (64 experts per pass).
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int64_t base = 0; base < a.E; base += 64) {
        const int64_t e = base + lane;
        int32_t lo = 0, hi = 0, nt = 0;
        if (e < a.E) {
            lo = a.offsets[e];
            hi = a.offsets[e + 1];
            nt = (hi - lo + BM - 1) / BM;
        }
        int32_t incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t up = __shfl_up(incl, d, 64);
            if (lane >= d) incl += up;
        }
        const int64_t first = acc + (incl - nt);
        const uint64_t hit = __ballot(e < a.E && tile >= first && tile < first + nt);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            // wave-uniform values, kept in scalar registers
            const int32_t lo_l = __builtin_amdgcn_readfirstlane(__shfl(lo, l, 64));
            const int32_t hi_l = __builtin_amdgcn_readfirstlane(__shfl(hi, l, 64));
            const int32_t first_l = __builtin_amdgcn_readfirstlane(__shfl((int32_t)(incl - nt), l, 64));
            tr.m0 = lo_l + (tile - acc - first_l) * BM;
            tr.m_end = hi_l;
            tr.expert = base + l;
            return true;
        }
        acc += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    }
    return false;
}

// Workgroups are dealt to the eight XCDs round-robin (id % 8).  Give each XCD
// a contiguous run of the tile order (token tiles fastest), so the tiles one
// XCD runs at the same time share weight and token rows in its own L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t wg, int64_t ntiles) {
    const int64_t per_xcd = (ntiles + 7) / 8;
    return (wg % 8) * per_xcd + wg / 8;
}

// Launches of several rounds of tiles: XCD x owns a band of RB row tiles and
// 1/G of the column tiles (G = 8 / bands, bands = n_mtiles / RB), row tiles
// fastest, so one band's token rows serve every column tile the XCD runs
// while its weight columns stream through (on MI355X at 2048 x 28672 x 4096,
// bands of two 256-row tiles: L2 hits up, 3% faster than column runs).
// Returns the tile index col * n_mtiles + row, or n_mtiles * n_ntiles past
// the XCD's share; the launcher sizes the grid as 8 * RB * ceil(n_ntiles / G).
__device__ __forceinline__ int64_t xcd_tile_band(int64_t wg, int64_t n_mtiles, int64_t n_ntiles, int64_t RB) {
    const int64_t G = 8 / (n_mtiles / RB);
    const int64_t x = wg % 8, q = wg / 8;
    const int64_t per = (n_ntiles + G - 1) / G;
    const int64_t col = (x % G) * per + q / RB;
    const int64_t row = (x / G) * RB + q % RB;
    if (q / RB >= per || col >= n_ntiles) return n_mtiles * n_ntiles;
    return col * n_mtiles + row;
}

// WGM x WGN waves: WGM along the token rows, WGN along the weight rows; NS
// LDS stages (2 or 3).
// LSPLIT (three stages only): the last LSPLIT of a stage's direct loads are
// issued one sub-step later than the rest, so the loads of all waves spread
// over a whole step instead of bunching in one sub-step.
// RPS LDS reads are issued per MFMA slot, so a sub-step's reads are all in
// flight early and have landed before the next sub-step needs them.
template <int FMT, int BM, int BN, int WGM, int WGN, int NS, int LSPLIT = 0, int RPS = 1>
struct DualGemm {
    static_assert(NS == 2 || NS == 3, "two or three stages");
    static_assert(LSPLIT == 0 || NS == 3, "split loads need a third stage");
    static constexpr int NW = WGM * WGN;
    using L = StageLayout<FMT, BM, BN, NW>;
    static constexpr int FM = BM / WGM / 32;  // 32-row token fragments per wave
    static constexpr int FN = BN / WGN / 32;  // 32-row weight fragments per wave

    // Operand fragments of one 64-wide sub-step, and the 16-bit scale pair
    // of every fragment row: MXFP4, blocks 2q and 2q+1 (byte T for sub-step
    // T, selected by opsel); NVFP4, the two 16-element blocks of unit 2q+T.
    struct Frags {
        v4i w[FN], xb[FM], xr[FM];
    };
    struct Scales {
        uint32_t w[FN], xb[FM], xr[FM];
    };

    __amdgpu_buffer_rsrc_t rW, rWs, rXb, rXr, rXbs, rXrs;
    uint32_t w_off[L::W_LD], x_off[L::X_LD], s_off[L::SC_LD];
    // NVFP4_SP24: the compressed backbone's rows are 48 bytes per stage (three
    // of the row's four 16-byte LDS units), so its loads have offsets of
    // their own
    uint32_t xb_off[FMT == kFmtNvSp ? L::X_LD : 1];
    // 16-row code load j of this wave: slot (wave * LD + j) mod the loads per
    // array (when the waves do not divide the loads evenly, the surplus ones
    // repeat a slot: identical bytes to identical places)
    static __device__ __forceinline__ int w_slot(int wave, int j) { return (wave * L::W_LD + j) % L::W_NI; }
    static __device__ __forceinline__ int x_slot(int wave, int j) { return (wave * L::X_LD + j) % L::X_NI; }
    // scale load k of this wave: resource, LDS offset in the stage, rows of
    // its array (wave-uniform, fixed at set-up so the K loop has no branches)
    __amdgpu_buffer_rsrc_t s_rsrc[L::SC_LD];
    int s_lds[L::SC_LD];
    uint32_t s_rows[L::SC_LD];
    int wave;  // wave-uniform
    int lane, wm, wn;
    int64_t last_step;
    uint32_t tw, tx;  // rows of the weight / token arrays: the K-tile stride

    // Scale-load instruction k of this wave: global index (wave + k*NW) mod
    // SC_TOT over [W chunks | XB chunks | XR chunks].
    static __device__ __forceinline__ int sc_index(int wave, int k) { return (wave + k * NW) % L::SC_TOT; }

    // One of this wave's PER_STAGE direct loads of stage `stage` into buffer
    // B (stages past the end reload the last one, so every step issues the
    // same number of loads).
    template <int B>
    __device__ __forceinline__ void issue_one(int idx, int64_t stage) {
        uint8_t *st = stage_buf<B, L::BYTES>();
        const int64_t stp = stage < last_step ? stage : last_step;
        if (idx < L::W_LD) {
            lds_load16(rW, st + L::W_CODES + w_slot(wave, idx) * 1024, w_off[idx],
                       (uint32_t)stp * tw * kRowBytes);
        } else if (idx < L::W_LD + 2 * L::X_LD) {
            const int j = (idx - L::W_LD) >> 1;
            const uint32_t cx = (uint32_t)stp * tx * kRowBytes;
            if (((idx - L::W_LD) & 1) == 0) {
                if constexpr (FMT == kFmtNvSp)
                    lds_load16(rXb, st + L::XB_CODES + x_slot(wave, j) * 1024, xb_off[j],
                               (uint32_t)stp * tx * kSpRowBytes);
                else
                    lds_load16(rXb, st + L::XB_CODES + x_slot(wave, j) * 1024, x_off[j], cx);
            } else {
                lds_load16(rXr, st + L::XR_CODES + x_slot(wave, j) * 1024, x_off[j], cx);
            }
        } else {
            const int k = idx - L::W_LD - 2 * L::X_LD;
            lds_load4(s_rsrc[k], st + s_lds[k], s_off[k], (uint32_t)stp * s_rows[k] * L::SB);
        }
    }

    template <int B>
    __device__ __forceinline__ void issue(int64_t stage) {
#pragma unroll
        for (int idx = 0; idx < L::PER_STAGE; idx++) issue_one<B>(idx, stage);
    }

    // Per-lane LDS byte offsets of the reads (row wn*FN*32 + l%32 for
    // weights, wm*FM*32 + l%32 for tokens; fragment j / i adds 32 rows, which
    // keeps the swizzle).
    int rd_w[2], rd_x[2], rd_ws[2], rd_xs[2];
    // NVFP4_SP24 backbone: the lane's 8 code bytes and index dword of
    // sub-step T (logical units T and 2 of its 48-byte row) and its scale
    // dword (the row's scales of units T and 2+T)
    int rd_xbc[2], rd_xbm[2], rd_xbs[2];

    __device__ __forceinline__ void init_reads() {
        const int frow = lane & 31, q = lane >> 5;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int sw = swz_unit(frow, 2 * q + t) * 16;
            rd_w[t] = (wn * (FN * 32) + frow) * kRowBytes + sw;
            rd_x[t] = (wm * (FM * 32) + frow) * kRowBytes + sw;
            const int sc = FMT == kFmtMx ? 2 * q : 2 * (2 * q + t);
            rd_ws[t] = (wn * (FN * 32) + frow) * L::SB + sc;
            rd_xs[t] = (wm * (FM * 32) + frow) * L::SB + sc;
            const int xrow = wm * (FM * 32) + frow;
            rd_xbc[t] = xrow * kRowBytes + swz_unit(frow, t) * 16 + 8 * q;
            rd_xbm[t] = xrow * kRowBytes + swz_unit(frow, 2) * 16 + 4 * (2 * t + q);
            rd_xbs[t] = xrow * L::SB + 4 * t;
        }
    }

    static constexpr int NREAD_FRAGS = FN + 2 * FM;
    static constexpr int NREAD_NEXT = 2 * NREAD_FRAGS;

    template <int B, int T>
    __device__ __forceinline__ void read_frag(int r, Frags &f) const {
        const uint8_t *cur = stage_buf<B, L::BYTES>();
        if (r < FN) {
            f.w[r] = *reinterpret_cast<const v4i *>(cur + (rd_w[T] + (L::W_CODES + r * 32 * kRowBytes)));
        } else {
            const int i = (r - FN) >> 1;
            if (((r - FN) & 1) == 0) {
                if constexpr (FMT == kFmtNvSp) {
                    const uint8_t *b = cur + L::XB_CODES + i * 32 * kRowBytes;
                    const uint2 c = *reinterpret_cast<const uint2 *>(b + rd_xbc[T]);
                    const uint32_t ix = *reinterpret_cast<const uint32_t *>(b + rd_xbm[T]);
                    f.xb[i] = v4i{(int)c.x, (int)c.y, (int)ix, 0};
                } else {
                    f.xb[i] = *reinterpret_cast<const v4i *>(cur + (rd_x[T] + (L::XB_CODES + i * 32 * kRowBytes)));
                }
            } else {
                f.xr[i] = *reinterpret_cast<const v4i *>(cur + (rd_x[T] + (L::XR_CODES + i * 32 * kRowBytes)));
            }
        }
    }

    template <int B, int T>
    __device__ __forceinline__ void read_scale(int r, Scales &s) const {
        const uint8_t *cur = stage_buf<B, L::BYTES>();
        if (r < FN) {
            s.w[r] = *reinterpret_cast<const uint16_t *>(cur + (rd_ws[T] + (L::W_SC + r * 32 * L::SB)));
        } else {
            const int i = (r - FN) >> 1;
            if (((r - FN) & 1) == 0) {
                if constexpr (FMT == kFmtNvSp)
                    s.xb[i] = *reinterpret_cast<const uint32_t *>(cur + (rd_xbs[T] + (L::XB_SC + i * 32 * L::SB)));
                else
                    s.xb[i] = *reinterpret_cast<const uint16_t *>(cur + (rd_xs[T] + (L::XB_SC + i * 32 * L::SB)));
            } else {
                s.xr[i] = *reinterpret_cast<const uint16_t *>(cur + (rd_xs[T] + (L::XR_SC + i * 32 * L::SB)));
            }
        }
    }

    // Read r of the next stage's first half, in the order the sub-step-0
    // MFMAs need them: each weight fragment's scale and codes, then per token
    // fragment the backbone and residual scales and codes.  NVFP4 reads the
    // sub-step-1 scales with the sub-step-1 fragments.
    template <int B>
    __device__ __forceinline__ void read_next(int r, Frags &f, Scales &s) const {
        if (r < 2 * FN) {
            if ((r & 1) == 0)
                read_scale<B, 0>(r >> 1, s);
            else
                read_frag<B, 0>(r >> 1, f);
        } else {
            const int i = (r - 2 * FN) >> 2, k = (r - 2 * FN) & 3;
            if (k < 2)
                read_scale<B, 0>(FN + 2 * i + k, s);
            else
                read_frag<B, 0>(FN + 2 * i + (k - 2), f);
        }
    }

    template <int B>
    __device__ __forceinline__ void read_sub1(int r, Frags &f, Scales &s) const {
        if (FMT == kFmtMx || r < NREAD_FRAGS)
            read_frag<B, 1>(r, f);
        else
            read_scale<B, 1>(r - NREAD_FRAGS, s);
    }

    // MFMAs of sub-step T, in the order (token fragment i, backbone then
    // residual, weight fragment j); so per accumulator: backbone then
    // residual, sub-step 0 then 1.
    //
    // Other work is threaded between the MFMAs, one piece after each, in
    // program order (scheduling barriers keep it there): MODE 0 reads the
    // sub-step-1 fragments (NVFP4: and scales) of buffer BR; MODE 1 reads the
    // scales and sub-step-0 fragments of buffer BR and, in the later slots,
    // issues the direct loads of stage `stage` into buffer BL.  A wave thus
    // never stalls behind a burst of memory instructions while its matrix
    // unit idles.
    template <int T, int MODE, int BL, int BR>
    __device__ __forceinline__ void mma(v16f (&acc)[FM][FN], const Frags &f, const Scales &s, int64_t stage,
                                        Frags &fo, Scales &so) {
        if constexpr (FMT == kFmtMx) {
            constexpr int NM = 2 * FM * FN;
            constexpr int NOTHER = MODE == 0 ? NREAD_FRAGS : NREAD_NEXT;
            // direct loads of this sub-step: indices [LLO, LLO + NLOAD)
            constexpr int NLOAD = MODE == 0 ? LSPLIT : L::PER_STAGE - LSPLIT;
            constexpr int LLO = MODE == 0 ? L::PER_STAGE - LSPLIT : 0;
            constexpr int NRSLOT = (NOTHER + RPS - 1) / RPS;
            constexpr int NSLOT = NM > NRSLOT ? (NM > NLOAD ? NM : NLOAD) : (NRSLOT > NLOAD ? NRSLOT : NLOAD);
#pragma unroll
            for (int k = 0; k < NSLOT; k++) {
                const int i = k / (2 * FN), p = (k / FN) & 1, j = k % FN;
                if (k < NM) {
                    if (p == 0)
                        acc[i][j] = mfma32_fp4<T>(f.w[j], f.xb[i], acc[i][j], (int)s.w[j], (int)s.xb[i]);
                    else
                        acc[i][j] = mfma32_fp4<T>(f.w[j], f.xr[i], acc[i][j], (int)s.w[j], (int)s.xr[i]);
                }
                if constexpr (LSPLIT == 0) {
                    constexpr int LOAD0 = NM > NLOAD ? NM - NLOAD - 1 : 0;  // loads go in the later slots
                    if (k >= LOAD0 && k - LOAD0 < NLOAD) this->template issue_one<BL>(k - LOAD0, stage);
                } else {
#pragma unroll
                    for (int l = 0; l < NLOAD; l++)  // spread evenly over the slots
                        if (((2 * l + 1) * NSLOT) / (2 * NLOAD) == k) this->template issue_one<BL>(LLO + l, stage);
                }
#pragma unroll
                for (int q = 0; q < RPS; q++) {
                    const int r = k * RPS + q;
                    if (r < NOTHER) {
                        if (MODE == 0)
                            read_sub1<BR>(r, fo, so);
                        else
                            read_next<BR>(r, fo, so);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (FMT == kFmtNvSp) {
            // NVFP4_SP24: per 32 K of a fragment pair one 2:4 sparse f16 MFMA
            // on the compressed backbone (eight kept values per lane) and two
            // dense f16 MFMAs on the residual, all three reading the same
            // dequantized weight half; the token fragment is the A operand
            // (accumulators hold token rows, see the epilogue).
            //
            // Per token fragment i, halves u = 0, 1 (K halves of the
            // sub-step).  The vector work runs one half ahead and is threaded
            // between the dense MFMAs of the current half (the sparse ones
            // are assembly, which the scheduler does not move): half (i, 0)
            // dequantizes half 1 of token fragment i (on i = 0 also half 1
            // of every weight fragment), half (i, 1) decodes the scales of
            // token fragment i+1 and dequantizes its half 0.
            constexpr int NOTHER = MODE == 0 ? 2 * NREAD_FRAGS : NREAD_NEXT;
            constexpr int NLOAD = MODE == 0 ? LSPLIT : L::PER_STAGE - LSPLIT;
            constexpr int LLO = MODE == 0 ? L::PER_STAGE - LSPLIT : 0;
            constexpr int PER_I_OTHER = (NOTHER + FM - 1) / FM;
            constexpr int PER_I_LOAD = (NLOAD + FM - 1) / FM;
            NvScale sw[FN], sxr[FM], sbl[FM], sbh[FM];
#pragma unroll
            for (int j = 0; j < FN; j++) sw[j] = nv_scale(s.w[j]);
            sxr[0] = nv_scale(s.xr[0]);
            sbl[0] = nv_scale(s.xb[0] & 0xFFFFu);
            sbh[0] = nv_scale(s.xb[0] >> 16);
            v16h wd[FN][2];
            v8h xb[2][2], xr[2][4];
#pragma unroll
            for (int j = 0; j < FN; j++)
                wd[j][0] = __builtin_shufflevector(nv_group<0>(f.w[j], sw[j]), nv_group<1>(f.w[j], sw[j]), 0, 1, 2,
                                                   3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
            xb[0][0] = sp_group<0>((uint32_t)f.xb[0].x, sbl[0], sbh[0]);
            xr[0][0] = nv_group<0>(f.xr[0], sxr[0]);
            xr[0][1] = nv_group<1>(f.xr[0], sxr[0]);
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int cb = i & 1;
                const uint32_t ix = (uint32_t)f.xb[i].z;
                auto half = [&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    // The sparse MFMAs first, fenced: the residual MFMAs on
                    // the same accumulators come FN matrix instructions later
                    // (with FN < 4 a pause pads the group).
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < FN; j++) {
                        if (j == 0)
                            smfmac32_f16<u, true>(acc[i][j], xb[cb][u], wd[j][u], ix);
                        else
                            smfmac32_f16<u, false>(acc[i][j], xb[cb][u], wd[j][u], ix);
                    }
                    if constexpr (FN < 4) asm volatile("s_nop 7\n\ts_nop 7");
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            xr[cb][2 * u], __builtin_shufflevector(wd[j][u], wd[j][u], 0, 1, 2, 3, 4, 5, 6, 7), acc[i][j],
                            0, 0, 0);
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            xr[cb][2 * u + 1],
                            __builtin_shufflevector(wd[j][u], wd[j][u], 8, 9, 10, 11, 12, 13, 14, 15), acc[i][j], 0, 0,
                            0);
                    // vector work for the next half
                    if constexpr (u == 0) {
                        if (i == 0) {
#pragma unroll
                            for (int j = 0; j < FN; j++)
                                wd[j][1] = __builtin_shufflevector(nv_group<2>(f.w[j], sw[j]), nv_group<3>(f.w[j], sw[j]),
                                                                   0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                        }
                        xb[cb][1] = sp_group<1>((uint32_t)f.xb[i].y, sbl[i], sbh[i]);
                        xr[cb][2] = nv_group<2>(f.xr[i], sxr[i]);
                        xr[cb][3] = nv_group<3>(f.xr[i], sxr[i]);
                    } else {
                        if (i + 1 < FM) {
                            sxr[i + 1] = nv_scale(s.xr[i + 1]);
                            sbl[i + 1] = nv_scale(s.xb[i + 1] & 0xFFFFu);
                            sbh[i + 1] = nv_scale(s.xb[i + 1] >> 16);
                            xb[cb ^ 1][0] = sp_group<0>((uint32_t)f.xb[i + 1].x, sbl[i + 1], sbh[i + 1]);
                            xr[cb ^ 1][0] = nv_group<0>(f.xr[i + 1], sxr[i + 1]);
                            xr[cb ^ 1][1] = nv_group<1>(f.xr[i + 1], sxr[i + 1]);
                        }
#pragma unroll
                        for (int k = i * PER_I_LOAD; k < (i + 1) * PER_I_LOAD && k < NLOAD; k++)
                            this->template issue_one<BL>(LLO + k, stage);
#pragma unroll
                        for (int k = i * PER_I_OTHER; k < (i + 1) * PER_I_OTHER && k < NOTHER; k++) {
                            if (MODE == 0)
                                read_sub1<BR>(k, fo, so);
                            else
                                read_next<BR>(k, fo, so);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 2 * FN; k++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                half(std::integral_constant<int, 0>{});
                half(std::integral_constant<int, 1>{});
            }
        } else {
            // NVFP4: dequantize each fragment once per sub-step, four f16
            // MFMAs per fragment pair; side work spread over the token
            // fragments.
            constexpr int NOTHER = MODE == 0 ? 2 * NREAD_FRAGS : NREAD_NEXT;
            constexpr int NLOAD = MODE == 0 ? LSPLIT : L::PER_STAGE - LSPLIT;
            constexpr int LLO = MODE == 0 ? L::PER_STAGE - LSPLIT : 0;
            constexpr int PER_I_OTHER = (NOTHER + FM - 1) / FM;
            constexpr int PER_I_LOAD = (NLOAD + FM - 1) / FM;
            // Software pipeline over groups of eight K elements: the scales
            // are decoded first, then group t+1 of the weight fragments (on
            // the first token fragment) and of the token fragments is
            // dequantized while the MFMAs of group t run.  Consecutive MFMAs
            // go to the FN different accumulators, so none waits on the
            // previous one.
            NvScale sw[FN], sxb[FM], sxr[FM];
#pragma unroll
            for (int j = 0; j < FN; j++) sw[j] = nv_scale(s.w[j]);
#pragma unroll
            for (int i = 0; i < FM; i++) {
                sxb[i] = nv_scale(s.xb[i]);
                sxr[i] = nv_scale(s.xr[i]);
            }
            v8h wd[FN][4], xb[2][4], xr[2][4];
#pragma unroll
            for (int j = 0; j < FN; j++) wd[j][0] = nv_group<0>(f.w[j], sw[j]);
            xb[0][0] = nv_group<0>(f.xb[0], sxb[0]);
            xr[0][0] = nv_group<0>(f.xr[0], sxr[0]);
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int cb = i & 1;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    if (t + 1 < 4) {
                        if (i == 0) {
#pragma unroll
                            for (int j = 0; j < FN; j++)
                                wd[j][t + 1] = t == 0 ? nv_group<1>(f.w[j], sw[j])
                                             : t == 1 ? nv_group<2>(f.w[j], sw[j]) : nv_group<3>(f.w[j], sw[j]);
                        }
                        xb[cb][t + 1] = t == 0 ? nv_group<1>(f.xb[i], sxb[i])
                                      : t == 1 ? nv_group<2>(f.xb[i], sxb[i]) : nv_group<3>(f.xb[i], sxb[i]);
                        xr[cb][t + 1] = t == 0 ? nv_group<1>(f.xr[i], sxr[i])
                                      : t == 1 ? nv_group<2>(f.xr[i], sxr[i]) : nv_group<3>(f.xr[i], sxr[i]);
                    } else if (i + 1 < FM) {
                        xb[cb ^ 1][0] = nv_group<0>(f.xb[i + 1], sxb[i + 1]);
                        xr[cb ^ 1][0] = nv_group<0>(f.xr[i + 1], sxr[i + 1]);
                    }
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wd[j][t], xb[cb][t], acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wd[j][t], xr[cb][t], acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int k = 0; k < 2 * FN; k++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                    }
                }
#pragma unroll
                for (int k = i * PER_I_LOAD; k < (i + 1) * PER_I_LOAD && k < NLOAD; k++)
                    this->template issue_one<BL>(LLO + k, stage);
#pragma unroll
                for (int k = i * PER_I_OTHER; k < (i + 1) * PER_I_OTHER && k < NOTHER; k++) {
                    if (MODE == 0)
                        read_sub1<BR>(k, fo, so);
                    else
                        read_next<BR>(k, fo, so);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Step s on buffer B.  On entry f0/sc hold stage s's sub-step-0
    // fragments and scales; on exit, stage s+1's.
    template <int B>
    __device__ __forceinline__ void step(int64_t s, v16f (&acc)[FM][FN], Frags &f0, Scales &sc) {
        Frags f1;
        Scales s1;  // NVFP4: sub-step-1 scales (MXFP4 uses sc for both sub-steps)
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 0 issues the late loads of stage s+2 (buffer (B+2)%3, read
        // last in step s-1, so free since that step's barrier)
        this->template mma<0, 0, NS == 3 ? (B + 2) % 3 : B, B>(acc, f0, sc, s + 2, f1, s1);
        wait_vmcnt<(NS - 2) * L::PER_STAGE, true>();  // own reads of stage s done, stage s+1 landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        Scales sn;
        this->template mma<1, 1, B, (B + 1) % NS>(acc, f1, FMT == kFmtMx ? sc : s1, s + NS, f0, sn);
        sc = sn;
    }
};

// Item q of XCD x's share of a grouped product: the tiles of experts x,
// x+8, x+16, ... in order, each expert's BM-row tiles times its n_ntiles
// column tiles (column tiles fastest).  The experts' tile counts are placed
// with a wave-wide prefix sum (64 experts per pass); false when q is past
// the end.  Wave-uniform results.
template <int BM>
__device__ __forceinline__ bool xcd_group_item(const LinearArgs &a, int xcd, int64_t q, int64_t n_ntiles,
                                               TileRows &tr, int64_t &nt) {
    const int lane = threadIdx.x & 63;
    const int64_t nexp = (a.E - xcd + 7) / 8;
    int64_t acc = 0;
    for (int64_t base = 0; base < nexp; base += 64) {
        const int64_t j = base + lane;
        int32_t lo = 0, hi = 0, ni = 0;
        if (j < nexp) {
            const int64_t e = xcd + 8 * j;
            lo = a.offsets[e];
            hi = a.offsets[e + 1];
            ni = (int32_t)(((hi - lo + BM - 1) / BM) * n_ntiles);
        }
        int32_t incl = ni;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t up = __shfl_up(incl, d, 64);
            if (lane >= d) incl += up;
        }
        const int64_t first = acc + (incl - ni);
        const uint64_t hit = __ballot(j < nexp && q >= first && q < first + ni);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            const int32_t lo_l = __builtin_amdgcn_readfirstlane(__shfl(lo, l, 64));
            const int32_t hi_l = __builtin_amdgcn_readfirstlane(__shfl(hi, l, 64));
            const int32_t first_l = __builtin_amdgcn_readfirstlane(__shfl((int32_t)(incl - ni), l, 64));
            const int64_t local = q - acc - first_l;
            nt = local % n_ntiles;
            tr.m0 = lo_l + (local / n_ntiles) * BM;
            tr.m_end = hi_l;
            tr.expert = xcd + 8 * (base + l);
            return true;
        }
        acc += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    }
    return false;
}

// SwiGLU epilogue (MXFP4): the tile's weight rows are gate/up pairs
// interleaved in 32-row groups (gate_up_row), so fragments 2p and 2p+1 of a
// wave hold gate and up of the same 32 hidden columns hc0 .. hc0+31 at the
// same accumulator positions: lane l, value 4q + e is column 8q + 4fq + e
// (fq = l / 32) of row l % 32, which makes the 32 columns one MX block held
// by lanes l and l ^ 32, sixteen values each, in four aligned groups of
// four.  Each value becomes x = fl32(SiLU(gate) * up) and the block is
// decomposed as the preparation operator does it (N:M mask, backbone codes
// and E8M0 scale, residual against the dequantized backbone, its codes and
// scale), then stored in the next linear's K-tiled layout (rows = a.rows,
// K = nout / 2): lane fq writes bytes 8fq .. 8fq+7 of the block's 16 code
// bytes of each path (the partner's nibbles come by one lane exchange),
// lane 0..31 the block's four mask bytes and the backbone scale, lane
// 32..63 the residual scale.
template <int M, int FM, int FN>
__device__ __forceinline__ void swiglu_epilogue(const LinearArgs &a, const v16f (&acc)[FM][FN], const TileRows &tr,
                                                int64_t n0, int lane, int wm, int wn) {
    static_assert(FN % 2 == 0, "gate/up fragment pairs");
    static_assert(M == 1 || M == 2 || M == 4, "mask groups inside the lane");
    const int frow = lane & 31, fq = lane >> 5;
    const int64_t Kd = a.nout / 2, Td = a.rows;
    const int64_t hb = (n0 + wn * (FN * 32)) / 2;  // hidden column of the wave's first pair
#pragma unroll
    for (int i = 0; i < FM; i++) {
        const int64_t m = tr.m0 + wm * (FM * 32) + i * 32 + frow;
        const bool row_ok = m < tr.m_end;
#pragma unroll
        for (int jp = 0; jp < FN / 2; jp++) {
            const int64_t hc0 = hb + jp * 32;
            if (hc0 >= Kd) continue;  // wave-uniform: columns past the product
            float gv[16], uv[16], h[16], S[16], dq[16], R[16];
#pragma unroll
            for (int k = 0; k < 16; k++) {
                gv[k] = acc[i][2 * jp][k];
                uv[k] = acc[i][2 * jp + 1][k];
            }
            silu_times_n<16>(gv, uv, h);
            uint32_t keep = 0;
            if (M == 4 && a.p_n == 2) {  // 2:4 on wave-wide lane masks (uniform branch)
                uint64_t km[16];
                select_2of4(h, km);
                select_2of4(h + 8, km + 8);
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    const bool b = __builtin_amdgcn_inverse_ballot_w64(km[k]);
                    S[k] = b ? h[k] : 0.0f;
                    keep |= (b ? 1u : 0u) << k;
                }
            } else {
                keep = select_in_lane<M>(h, a.p_n) | (select_in_lane<M>(h + 8, a.p_n) << 8);
#pragma unroll
                for (int k = 0; k < 16; k++) S[k] = (keep >> k) & 1u ? h[k] : 0.0f;
            }
            float am = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; k++) am = fmaxf(am, fabsf(S[k]));
            am = fmaxf(am, __shfl_xor(am, 32, 64));
            const int Eb = mx_shared_exp(am);
            const float sb = e8m0_operand(Eb);
            const uint32_t bc0 = e2m1_cvt8(S, sb), bc1 = e2m1_cvt8(S + 8, sb);
            e2m1_dec8(bc0, sb, dq);
            e2m1_dec8(bc1, sb, dq + 8);
            float ar = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; k++) {
                R[k] = __fsub_rn(h[k], dq[k]);
                ar = fmaxf(ar, fabsf(R[k]));
            }
            ar = fmaxf(ar, __shfl_xor(ar, 32, 64));
            const int Er = mx_shared_exp(ar);
            const float sr = e8m0_operand(Er);
            const uint32_t rc0 = e2m1_cvt8(R, sr), rc1 = e2m1_cvt8(R + 8, sr);
            // block code bytes: lane fq = 0 holds columns 0-3, 8-11 (bc0) and
            // 16-19, 24-27 (bc1), lane fq = 1 columns 4-7, 12-15, 20-23, 28-31
            const uint32_t bx = __shfl_xor(fq ? bc0 : bc1, 32, 64);
            const uint32_t rx = __shfl_xor(fq ? rc0 : rc1, 32, 64);
            const uint32_t bl = fq ? bx : bc0, bh = fq ? bc1 : bx;  // words of lane 0..31 / 32..63
            const uint32_t rl = fq ? rx : rc0, rh = fq ? rc1 : rx;
            const uint2 bw = make_uint2((bl & 0xFFFFu) | (bh << 16), (bl >> 16) | (bh & 0xFFFF0000u));
            const uint2 rw = make_uint2((rl & 0xFFFFu) | (rh << 16), (rl >> 16) | (rh & 0xFFFF0000u));
            // mask: byte q of the block = nibble q of lane fq = 0 | nibble q of lane fq = 1 << 4
            const uint32_t sp = (keep & 0xFu) | ((keep & 0xF0u) << 4) | ((keep & 0xF00u) << 8) | ((keep & 0xF000u) << 12);
            const uint32_t mw = sp | (__shfl_xor(sp, 32, 64) << 4);
            if (row_ok) {
                const int64_t kt = hc0 / kTileK;
                const int64_t co = kt * Td * (kTileK / 2) + m * (kTileK / 2) + (hc0 % kTileK) / 2 + 8 * fq;
                *reinterpret_cast<uint2 *>(a.p_b_codes + co) = bw;
                *reinterpret_cast<uint2 *>(a.p_r_codes + co) = rw;
                const int64_t so = kt * Td * (kTileK / 32) + m * (kTileK / 32) + (hc0 % kTileK) / 32;
                if (fq == 0) {
                    a.p_b_scales[so] = (uint8_t)(Eb + 127);
                    if (a.p_mask) *reinterpret_cast<uint32_t *>(a.p_mask + m * (Kd / 8) + hc0 / 8) = mw;
                } else {
                    a.p_r_scales[so] = (uint8_t)(Er + 127);
                }
            }
        }
    }
}

// One BM x BN output tile: rows tr.m0 .. min(tr.m0 + BM, tr.m_end) - 1 of
// expert tr.expert, columns n0 .. n0 + BN - 1.
// EPI = 0: the product to y; EPI = M (1, 2 or 4): the SwiGLU epilogue with
// M-element mask groups (MXFP4), and the product to y when y is not null.
template <int FMT, int BM, int BN, int WGM, int WGN, int NS, int OCC, int LSPLIT, int RPS, int EPI = 0>
__device__ __forceinline__ void dual_tile(const LinearArgs &a, const TileRows &tr, int64_t n0) {
    using G = DualGemm<FMT, BM, BN, WGM, WGN, NS, LSPLIT, RPS>;
    using L = typename G::L;
    constexpr int FM = G::FM, FN = G::FN;
    static_assert(FM >= 1 && FN >= 1, "tile too small for 32x32 fragments");
    const int64_t K = a.K;
    constexpr int SB = L::SB;
    const uint32_t kb = (uint32_t)(K / 2), ks = (uint32_t)(K / kKS) * SB;  // per row: code / scale bytes
    const uint32_t nout = (uint32_t)a.nout;

    G g;
    g.rW = make_rsrc(a.w_codes + tr.expert * a.nout * kb, nout * kb);
    g.rWs = make_rsrc(a.w_scales + tr.expert * a.nout * ks, nout * ks);
    const uint32_t kbb = FMT == kFmtNvSp ? (uint32_t)(K / kKS) * kSpRowBytes : kb;  // backbone bytes per row
    g.rXb = make_rsrc(a.b_codes, (uint32_t)a.T * kbb);
    g.rXr = make_rsrc(a.r_codes, (uint32_t)a.T * kb);
    g.rXbs = make_rsrc(a.b_scales, (uint32_t)a.T * ks);
    g.rXrs = make_rsrc(a.r_scales, (uint32_t)a.T * ks);
    const int tid = threadIdx.x;
    g.lane = tid & 63;
    g.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    g.wm = g.wave / WGN;
    g.wn = g.wave % WGN;
    g.last_step = K / kKS - 1;
    g.tw = nout;
    g.tx = (uint32_t)a.T;
    g.init_reads();

    // source offsets of the slots this lane fills (fixed over K)
#pragma unroll
    for (int j = 0; j < L::W_LD; j++) {
        const int row = G::w_slot(g.wave, j) * 16 + (g.lane >> 2);
        const int unit = swz_unit(row, g.lane & 3);
        const int64_t n = n0 + row;
        g.w_off[j] = n < a.nout ? (uint32_t)n * kRowBytes + unit * 16 : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < L::X_LD; j++) {
        const int row = G::x_slot(g.wave, j) * 16 + (g.lane >> 2);
        const int unit = swz_unit(row, g.lane & 3);
        const int64_t m = tr.m0 + row;
        const int64_t src = m < tr.m_end ? (a.row_index ? (int64_t)a.row_index[m] : m) : -1;
        g.x_off[j] = src >= 0 ? (uint32_t)src * kRowBytes + unit * 16 : kOutOfRange;
        if constexpr (FMT == kFmtNvSp)  // units 0-2 of the 48-byte row; LDS unit 3 stays zero
            g.xb_off[j] = src >= 0 && unit < 3 ? (uint32_t)src * kSpRowBytes + unit * 16 : kOutOfRange;
    }
    // scale slots: 4 bytes per lane, SB/4 lanes per row
#pragma unroll
    for (int k = 0; k < L::SC_LD; k++) {
        const int gi = G::sc_index(g.wave, k);
        const int lpr = SB / 4;
        const int part = (g.lane % lpr) * 4;
        if (gi < L::SC_W) {
            const int64_t n = n0 + gi * L::RPI + g.lane / lpr;
            g.s_off[k] = n < a.nout ? (uint32_t)n * SB + part : kOutOfRange;
            g.s_rsrc[k] = g.rWs;
            g.s_lds[k] = L::W_SC + gi * 256;
            g.s_rows[k] = nout;
        } else {
            const int c = (gi - L::SC_W) % L::SC_X;
            const int64_t m = tr.m0 + c * L::RPI + g.lane / lpr;
            const int64_t src = m < tr.m_end ? (a.row_index ? (int64_t)a.row_index[m] : m) : -1;
            g.s_off[k] = src >= 0 ? (uint32_t)src * SB + part : kOutOfRange;
            const bool resid = gi >= L::SC_W + L::SC_X;
            g.s_rsrc[k] = resid ? g.rXrs : g.rXbs;
            g.s_lds[k] = (resid ? L::XR_SC : L::XB_SC) + c * 256;
            g.s_rows[k] = (uint32_t)a.T;
        }
    }

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int64_t nsteps = K / kKS;
    typename G::Frags f0;
    typename G::Scales sc;
    g.template issue<0>(0);
    g.template issue<1>(1);
    if constexpr (NS == 3) {  // stage 2 less its late loads (issued in step 0)
#pragma unroll
        for (int idx = 0; idx < L::PER_STAGE - LSPLIT; idx++) g.template issue_one<2>(idx, 2);
    }
    wait_vmcnt<(NS - 1) * L::PER_STAGE - LSPLIT>();  // stage 0 landed
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < G::NREAD_NEXT; r++) g.template read_next<0>(r, f0, sc);
    int64_t s = 0;
    for (; s + NS <= nsteps; s += NS) {
        g.template step<0>(s, acc, f0, sc);
        g.template step<1>(s + 1, acc, f0, sc);
        if constexpr (NS == 3) g.template step<2>(s + 2, acc, f0, sc);
    }
    if (s < nsteps) g.template step<0>(s, acc, f0, sc);
    if (NS == 3 && s + 1 < nsteps) g.template step<1>(s + 1, acc, f0, sc);
    wait_vmcnt<0, true>();  // drain the tail loads before the workgroup exits

    // ---- epilogue: accumulator group q of fragment (i, j) is Y[m][n..n+3];
    // NVFP4 applies the two tensor scales here
    float alpha = 1.0f;
    if constexpr (FMT != kFmtMx) alpha = __fmul_rn(*a.x_gscale, a.w_gscale[tr.expert]);
    const int frow = g.lane & 31, fq = g.lane >> 5;
    const int wm = g.wm, wn = g.wn;
    if constexpr (FMT == kFmtNvSp) {
        // token fragments were the A operand: accumulator r of fragment (i, j)
        // is Y[m][n] with m = row 8(r/4) + 4*fq + r%4 of the token fragment
        // and n = column frow of the weight fragment
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int64_t n = n0 + wn * (FN * 32) + j * 32 + frow;
                if (n >= a.nout) continue;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t m = tr.m0 + wm * (FM * 32) + i * 32 + 8 * (r / 4) + 4 * fq + (r % 4);
                    if (m < tr.m_end) store_out1(a, m, n, __fmul_rn(acc[i][j][r], alpha));
                }
            }
        }
        return;
    }
    if (EPI == 0 || a.y != nullptr) {
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int64_t m = tr.m0 + wm * (FM * 32) + i * 32 + frow;
            if (m >= tr.m_end) continue;
#pragma unroll
            for (int j = 0; j < FN; j++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int64_t n = n0 + wn * (FN * 32) + j * 32 + 8 * q + 4 * fq;
                    v4f v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    if constexpr (FMT != kFmtMx) v = v4f{__fmul_rn(v.x, alpha), __fmul_rn(v.y, alpha),
                                                         __fmul_rn(v.z, alpha), __fmul_rn(v.w, alpha)};
                    store_out4(a, m, n, v);
                }
            }
        }
    }
    if constexpr (EPI != 0) {
        static_assert(FMT == kFmtMx, "the SwiGLU epilogue is MXFP4");
        swiglu_epilogue<EPI, FM, FN>(a, acc, tr, n0, g.lane, wm, wn);
    }
}


// A grid of tiles: dense products map blockIdx.x to a tile in XCD-aware
// order; grouped products either find their expert tile from blockIdx.x
// (n_mtiles = 0) or, as persistent workgroups (n_mtiles < 0), walk their
// XCD's share of the expert tiles (see xcd_group_item), so that the tiles of
// one expert run together on one XCD and share its weight and token rows in
// that XCD's L2.  OCC workgroups share a CU (LDS and registers are sized for
// that).
template <int FMT, int BM, int BN, int WGM, int WGN, int NS, int OCC, int LSPLIT, int RPS, bool GROUPED, int EPI>
__global__ __launch_bounds__(WGM * WGN * 64)
__attribute__((amdgpu_waves_per_eu(OCC * WGM * WGN / 4, OCC * WGM * WGN / 4)))
void k_dual_gemm(LinearArgs a, int64_t n_ntiles, int64_t n_mtiles, int64_t n_begin) {
    if (a.ksplit_tiles > 0) {  // MXFP4 only
        // K range blockIdx.y: in the K-tiled layout tiles [t0, t0 + kt) of every
        // operand are themselves a K-tiled array with K = 128 * kt
        constexpr int64_t kScaleBytes = kTileK / (FMT == kFmtMx ? 32 : 16);  // per row and K tile
        const int64_t t0 = (int64_t)blockIdx.y * a.ksplit_tiles;
        a.b_codes += t0 * a.T * (kTileK / 2);
        a.r_codes += t0 * a.T * (kTileK / 2);
        a.b_scales += t0 * a.T * kScaleBytes;
        a.r_scales += t0 * a.T * kScaleBytes;
        a.w_codes += t0 * a.nout * (kTileK / 2);
        a.w_scales += t0 * a.nout * kScaleBytes;
        a.K = a.ksplit_tiles * kTileK;
        a.y = static_cast<float *>(a.y) + (int64_t)blockIdx.y * a.split_stride;  // FP32 partials
    }
    using L = typename DualGemm<FMT, BM, BN, WGM, WGN, NS, LSPLIT, RPS>::L;
    static_assert(L::BYTES * NS * OCC <= kLdsBytes, "stages do not fit the CU's LDS");
    if constexpr (!GROUPED) {
        const int64_t t = a.xcd_band > 0 ? xcd_tile_band(blockIdx.x, n_mtiles, n_ntiles, a.xcd_band)
                                         : xcd_tile(blockIdx.x, n_ntiles * n_mtiles);
        if (t >= n_ntiles * n_mtiles) return;
        TileRows tr;
        tr.m0 = (t % n_mtiles) * BM;
        tr.m_end = a.rows;
        tr.expert = 0;
        dual_tile<FMT, BM, BN, WGM, WGN, NS, OCC, LSPLIT, RPS, EPI>(a, tr, n_begin + (t / n_mtiles) * BN);
        return;
    }
    // grouped: one tile found from blockIdx.x, or a persistent walk over
    // this XCD's tiles; a single call site keeps the tile inlined
    const bool persistent = n_mtiles < 0;
    for (int64_t q = blockIdx.x / 8;; q += gridDim.x / 8) {
        TileRows tr;
        int64_t n0;
        if (persistent) {
            int64_t nt;
            if (!xcd_group_item<BM>(a, (int)(blockIdx.x % 8), q, n_ntiles, tr, nt)) return;
            n0 = n_begin + nt * BN;
            __syncthreads();  // every wave is done with the previous tile's LDS stages
        } else {
            if (!grouped_tile_rows<BM>(a, blockIdx.x / n_ntiles, tr)) return;
            n0 = n_begin + (blockIdx.x % n_ntiles) * BN;
        }
        dual_tile<FMT, BM, BN, WGM, WGN, NS, OCC, LSPLIT, RPS, EPI>(a, tr, n0);
        if (!persistent) return;
    }
}
// ============================================================================
// Decode / small-T.  A workgroup of kSmallWaves waves owns 16 weight rows and
// splits K between its waves (wave w takes the w-th contiguous share of the
// 512-element K chunks); lane (r = l%16, q = l/16) streams the 64 code bytes
// and the scale dword of weight row r in K tile 4c+q of chunk c, so quarter q
// feeds blocks 4q..4q+3 and MFMA j (opsel j) uses block 4q+j.  In the K-tiled
// layout the 16 rows of one quarter are one contiguous kilobyte.  Token rows
// come the same way (they are few and stay in L2).  Each wave loads its next
// weight chunk before it multiplies the current one; the waves' partial sums meet in
// LDS and are added in wave order, so the result does not depend on timing.
// ============================================================================
constexpr int kSmallWaves = 8;
constexpr int kChunkK = 512;

struct Chunk64 {
    uint4 u[4];
    uint32_t sc;
};

// 64 code bytes and one scale dword of K tile 4c+q for the lane's row
// (code_row = row * 64, sc_row = row * 4, or kOutOfRange; `rows` rows per
// tile); rows or tiles that do not exist read as zeros (zero codes
// contribute nothing whatever the scale).
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                           uint32_t code_row, uint32_t sc_row, uint32_t rows, int64_t c,
                                           int q, int64_t K, Chunk64 &o) {
    const int64_t tile = c * (kChunkK / kTileK) + q;
    const bool in = tile * kTileK < K;
    const uint32_t co = in ? code_row + (uint32_t)tile * rows * (kTileK / 2) : kOutOfRange;
    const uint32_t so = in ? sc_row + (uint32_t)tile * rows * (kTileK / 32) : kOutOfRange;
    o.u[0] = bload128(rc, co);
    o.u[1] = bload128(rc, co + 16);
    o.u[2] = bload128(rc, co + 32);
    o.u[3] = bload128(rc, co + 48);
    o.sc = bload32(rs, so);
}

__device__ __forceinline__ v4i as_v4i(uint4 u) { return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}; }

template <int FM>
struct SmallGemm {
    __amdgpu_buffer_rsrc_t rW, rWs, rXb, rXr, rXbs, rXrs;
    uint32_t wrow, wsrow, x_row[FM], xs_row[FM];
    uint32_t nout, T;
    int q;
    int64_t K;

    __device__ __forceinline__ void load_w(int64_t c, Chunk64 &w) const {
        load_chunk(rW, rWs, wrow, wsrow, nout, c, q, K, w);
    }

    // the token rows' chunk c (few rows, L2-resident) and the MFMAs with the
    // weight chunk w
    __device__ __forceinline__ void mma(int64_t c, const Chunk64 &w, v4f (&acc)[FM]) const {
        Chunk64 xb[FM], xr[FM];
#pragma unroll
        for (int f = 0; f < FM; f++) {
            load_chunk(rXb, rXbs, x_row[f], xs_row[f], T, c, q, K, xb[f]);
            load_chunk(rXr, rXrs, x_row[f], xs_row[f], T, c, q, K, xr[f]);
        }
#pragma unroll
        for (int f = 0; f < FM; f++) {
            const Chunk64 &b = xb[f], &r = xr[f];
            acc[f] = mfma_fp4_sel<0>(as_v4i(w.u[0]), as_v4i(b.u[0]), acc[f], (int)w.sc, (int)b.sc);
            acc[f] = mfma_fp4_sel<0>(as_v4i(w.u[0]), as_v4i(r.u[0]), acc[f], (int)w.sc, (int)r.sc);
            acc[f] = mfma_fp4_sel<1>(as_v4i(w.u[1]), as_v4i(b.u[1]), acc[f], (int)w.sc, (int)b.sc);
            acc[f] = mfma_fp4_sel<1>(as_v4i(w.u[1]), as_v4i(r.u[1]), acc[f], (int)w.sc, (int)r.sc);
            acc[f] = mfma_fp4_sel<2>(as_v4i(w.u[2]), as_v4i(b.u[2]), acc[f], (int)w.sc, (int)b.sc);
            acc[f] = mfma_fp4_sel<2>(as_v4i(w.u[2]), as_v4i(r.u[2]), acc[f], (int)w.sc, (int)r.sc);
            acc[f] = mfma_fp4_sel<3>(as_v4i(w.u[3]), as_v4i(b.u[3]), acc[f], (int)w.sc, (int)b.sc);
            acc[f] = mfma_fp4_sel<3>(as_v4i(w.u[3]), as_v4i(r.u[3]), acc[f], (int)w.sc, (int)r.sc);
        }
    }
};

template <int FM>
__global__ __launch_bounds__(kSmallWaves * 64) void k_dual_gemm_mx_small(LinearArgs a) {
    __shared__ v4f part[kSmallWaves][FM][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t K = a.K, kb = K / 2, ks = K / 32;
    const int64_t nch = (K + kChunkK - 1) / kChunkK;
    const int64_t cpw = (nch + kSmallWaves - 1) / kSmallWaves;
    const int64_t c0 = wave * cpw;
    const int64_t c1 = c0 + cpw < nch ? c0 + cpw : nch;

    SmallGemm<FM> g;
    g.rW = make_rsrc(a.w_codes, (uint32_t)(a.nout * kb));
    g.rWs = make_rsrc(a.w_scales, (uint32_t)(a.nout * ks));
    g.rXb = make_rsrc(a.b_codes, (uint32_t)(a.T * kb));
    g.rXr = make_rsrc(a.r_codes, (uint32_t)(a.T * kb));
    g.rXbs = make_rsrc(a.b_scales, (uint32_t)(a.T * ks));
    g.rXrs = make_rsrc(a.r_scales, (uint32_t)(a.T * ks));
    g.nout = (uint32_t)a.nout;
    g.T = (uint32_t)a.T;
    g.q = lane >> 4;
    g.K = K;
    const bool wvalid = n0 + r < a.nout;
    g.wrow = wvalid ? (uint32_t)((n0 + r) * (kTileK / 2)) : kOutOfRange;
    g.wsrow = wvalid ? (uint32_t)((n0 + r) * (kTileK / 32)) : kOutOfRange;
#pragma unroll
    for (int f = 0; f < FM; f++) {
        const int64_t m = f * 16 + r;
        const int64_t src = m < a.rows ? (a.row_index ? (int64_t)a.row_index[m] : m) : -1;
        g.x_row[f] = src >= 0 ? (uint32_t)(src * (kTileK / 2)) : kOutOfRange;
        g.xs_row[f] = src >= 0 ? (uint32_t)(src * (kTileK / 32)) : kOutOfRange;
    }

    v4f acc[FM];
#pragma unroll
    for (int f = 0; f < FM; f++) acc[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // two weight chunks in flight: the next one loads while the current one
    // multiplies
    Chunk64 wa, wb;
    if (c0 < c1) g.load_w(c0, wa);
    for (int64_t c = c0; c < c1; c += 2) {
        if (c + 1 < c1) g.load_w(c + 1, wb);
        g.mma(c, wa, acc);
        if (c + 2 < c1) g.load_w(c + 2, wa);
        if (c + 1 < c1) g.mma(c + 1, wb, acc);
    }

#pragma unroll
    for (int f = 0; f < FM; f++) part[wave][f][lane] = acc[f];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int f = 0; f < FM; f++) {
        v4f s = part[0][f][lane];
#pragma unroll
        for (int w = 1; w < kSmallWaves; w++) {
            const v4f p = part[w][f][lane];
            s = v4f{__fadd_rn(s.x, p.x), __fadd_rn(s.y, p.y), __fadd_rn(s.z, p.z), __fadd_rn(s.w, p.w)};
        }
        const int64_t m = f * 16 + r;
        if (m >= a.rows) continue;
        store_out4(a, m, n0 + (lane >> 4) * 4, s);
    }
}

// ============================================================================
// launcher
// ============================================================================
static int device_cus();

// Output columns [n_begin, n_end) of the product (all of them by default).
// Grouped products: `persistent` launches OCC workgroups per CU that walk
// their XCD's share of the expert tiles; otherwise one workgroup per tile
// (an upper bound of tiles is launched, the extra workgroups exit).
template <int FMT, int BM, int BN, int WGM, int WGN, int NS = 3, int OCC = 1, int LSPLIT = 0, int RPS = 1,
          bool GROUPED = false, int EPI = 0>
static hipError_t launch_prefill(const LinearArgs &a, hipStream_t st, int64_t n_begin = 0, int64_t n_end = -1,
                                 bool persistent = false) {
    if (n_end < 0) n_end = a.nout;
    const int64_t n_ntiles = (n_end - n_begin + BN - 1) / BN;
    int64_t blocks;
    int64_t n_mtiles = 0;
    LinearArgs ab = a;
    ab.xcd_band = 0;
    if (a.offsets && persistent) {
        blocks = (int64_t)((device_cus() + 7) / 8) * 8 * OCC;
        n_mtiles = -1;
    } else if (a.offsets) {
        blocks = n_ntiles * ((a.rows + BM - 1) / BM + a.E);  // upper bound; extra blocks exit
    } else {
        n_mtiles = (a.rows + BM - 1) / BM;
        blocks = ((n_ntiles * n_mtiles + 7) / 8) * 8;
        // MXFP4 launches of more than one round: XCD bands of 512 token rows,
        // when 2 or 4 bands split the rows (each band then shared by 4 or 2
        // XCDs, so no XCD streams the whole weight)
        constexpr int64_t RB = BM >= 512 ? 1 : 512 / BM;
        if (FMT == kFmtMx && a.ksplit_tiles == 0 && n_ntiles * n_mtiles > (int64_t)device_cus() * OCC &&
            (n_mtiles == 2 * RB || n_mtiles == 4 * RB)) {
            const int64_t G = 8 / (n_mtiles / RB);
            ab.xcd_band = RB;
            blocks = 8 * RB * ((n_ntiles + G - 1) / G);
        }
    }
    const unsigned splits = a.ksplit_tiles > 0 ? (unsigned)(a.K / kTileK / a.ksplit_tiles) : 1u;
    hipLaunchKernelGGL((k_dual_gemm<FMT, BM, BN, WGM, WGN, NS, OCC, LSPLIT, RPS, GROUPED, EPI>), dim3((unsigned)blocks, splits),
                       dim3(WGM * WGN * 64), 0,
                       st, ab, n_ntiles, n_mtiles, n_begin);
    return hipGetLastError();
}

template <int FM>
static hipError_t launch_small(const LinearArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((k_dual_gemm_mx_small<FM>), dim3((unsigned)((a.nout + 15) / 16)), dim3(kSmallWaves * 64), 0, st,
                       a);
    return hipGetLastError();
}

// Compute units of the current device (cached per device id).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Dense MXFP4 tile shapes: 256x256 and 256x192 (8 waves), 128x256 and 128x128
// (4 waves).
// One workgroup fills a CU (LDS), so a launch takes about rounds(tiles / CUs)
// times the tile time, with smaller tiles paying for their lower operand
// reuse (relative cost per output element, measured on MI355X for
// K = 4096..14336).
struct TileShape {
    int bm, bn;
    double cost;
};
constexpr int kNumMxShapes = 4;
constexpr TileShape kMxShapes[kNumMxShapes] = {{256, 256, 1.0}, {128, 256, 1.2}, {128, 128, 1.5}, {256, 192, 1.27}};

static double shape_time(int s, int64_t rows, int64_t cols, int64_t cus) {
    const TileShape &t = kMxShapes[s];
    const int64_t tiles = ((rows + t.bm - 1) / t.bm) * ((cols + t.bn - 1) / t.bn);
    return (double)((tiles + cus - 1) / cus) * t.bm * t.bn * t.cost;
}

// Fastest shape by the model; even_fn: only shapes whose waves hold an even
// number of 32-column fragments (the SwiGLU epilogue's gate/up pairs).
static int best_shape(int64_t rows, int64_t cols, int64_t cus, double *t_best, bool even_fn = false) {
    int best = 0;
    for (int s = 0; s < kNumMxShapes; s++) {
        if (even_fn && s == 3) continue;  // 256x192: three fragments per wave
        const double t = shape_time(s, rows, cols, cus);
        if (s == 0 || t < *t_best) {
            best = s;
            *t_best = t;
        }
    }
    return best;
}

template <int EPI = 0>
static hipError_t launch_mx_shape(int s, const LinearArgs &a, hipStream_t st, int64_t n_begin, int64_t n_end) {
    // split loads over two sub-steps, two LDS reads per MFMA slot
    if (s == 0) return launch_prefill<kFmtMx, 256, 256, 4, 2, 3, 1, 4, 2, false, EPI>(a, st, n_begin, n_end);
    if (s == 1) return launch_prefill<kFmtMx, 128, 256, 2, 2, 3, 1, 4, 2, false, EPI>(a, st, n_begin, n_end);
    if constexpr (EPI == 0)
        if (s == 3) return launch_prefill<kFmtMx, 256, 192, 4, 2, 3, 1, 4, 2>(a, st, n_begin, n_end);
    return launch_prefill<kFmtMx, 128, 128, 2, 2, 3, 1, 0, 1, false, EPI>(a, st, n_begin, n_end);
}

// A product whose 256x256 tiles fill some rounds of the CUs and leave a
// partial last round runs as two launches over column ranges: full rounds
// of 256x256 tiles, then the remaining columns in the shape that fits them
// best, instead of a last round that leaves CUs idle.
// Sum of S partial products p[S][rows][nout] (row-major FP32) into y, the
// partials added in the order s = 0, 1, ..., S-1.
// The sum is stored in the output type of the product.
__global__ __launch_bounds__(256) void k_sum_partials(const float *p, int S, int64_t rows, int64_t nout, void *y,
                                                      int ydt, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t plane = rows * nout;
    if (i >= plane) return;
    const int64_t m = i / nout, n = i - m * nout;
    float acc = p[i];
    for (int s = 1; s < S; s++) acc = __fadd_rn(acc, p[(int64_t)s * plane + i]);
    if (ydt == kOutF32)
        static_cast<float *>(y)[m * ldy + n] = acc;
    else
        static_cast<uint16_t *>(y)[m * ldy + n] = (uint16_t)out_bits16(acc, ydt);
}

// Up to 64 rows: the small-batch kernel (weight rows split over many
// workgroups, K over their waves; every workgroup re-reads the token rows),
// one row of 64x64 tiles with two workgroups per CU, or those tiles over S
// equal K ranges (S independent products into the workspace, then summed
// in a fixed order), whichever this model of MI355X measurements says is
// fastest (times in us): the small kernel streams the weight at about
// 3.5 / 2.2 / 1.6 / 1.2 TB/s for 16 / 32 / 48 / 64 rows after about 3 us;
// the tiles take about 0.31 us per 128-wide K step and round of tiles (two
// per CU), or stream the weight at 4.5 TB/s, after about 1 us; a K split
// adds the summing pass (about 4 us plus the partials' traffic at 3 TB/s)
// and is taken only when it is 10% faster.  K splits are used from 17 rows on, in one launch whose second
// grid dimension is the K range.  The model assumes the MI355X's 256 CUs,
// so that the workspace size does not depend on the device.
constexpr int64_t kFewRowsModelCus = 256;

struct FewRowsPlan {
    int kernel;  // 0 small-batch kernel, 1 64x64 tiles, 2 64x64 tiles over S K ranges
    int S;
};

static FewRowsPlan plan_few_rows(int64_t rows, int64_t K, int64_t nout) {
    constexpr double kSmallTBps[4] = {3.5, 2.2, 1.6, 1.2};
    const int fm = rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 48 ? 3 : 4;
    const double w_mb = (double)nout * (double)K * (0.5 + 1.0 / 32.0) * 1e-6;
    const int64_t tiles = (nout + 63) / 64, slots = 2 * kFewRowsModelCus, ksteps = K / 128;
    auto t_tiles = [&](int S) {
        const double rounds = (double)((tiles * S + slots - 1) / slots);
        const double t_step = (double)(ksteps / S) * 0.31 * rounds, t_stream = w_mb / 4.5;
        const double t = 1.0 + (t_step > t_stream ? t_step : t_stream);
        // partials written once and read once, the sum written, at 3 TB/s
        return S == 1 ? t : t + 4.0 + (double)(2 * S + 1) * (double)rows * (double)nout * 4.0 * 1e-6 / 3.0;
    };
    FewRowsPlan best{0, 1};
    double t_best = 3.0 + w_mb / kSmallTBps[fm - 1];
    if (t_tiles(1) < t_best) {
        best = {1, 1};
        t_best = t_tiles(1);
    }
    if (rows > 16) {
        for (int S = 2; S <= 8; S *= 2) {
            if (ksteps % S != 0 || ksteps / S < 4) continue;
            const double t = t_tiles(S);
            if (t < 0.9 * t_best) {  // only a clear gain pays for the extra pass
                best = {2, S};
                t_best = t;
            }
        }
    }
    return best;
}

static size_t few_rows_workspace(int64_t rows, int64_t K, int64_t nout) {
    const FewRowsPlan pl = plan_few_rows(rows, K, nout);
    return pl.kernel == 2 ? (size_t)pl.S * (size_t)rows * (size_t)nout * sizeof(float) : 0;
}

static hipError_t launch_linear_mx_few_rows(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st) {
    const FewRowsPlan pl = plan_few_rows(a.rows, a.K, a.nout);
    if (pl.kernel == 2 && ws != nullptr && ws_bytes >= few_rows_workspace(a.rows, a.K, a.nout)) {
        // one launch: grid row s multiplies K range s into partial product s
        float *part = static_cast<float *>(ws);
        LinearArgs as = a;
        as.ksplit_tiles = a.K / kTileK / pl.S;
        as.split_stride = a.rows * a.nout;
        as.y = part;
        as.ydt = kOutF32;
        as.ldy = a.nout;
        as.y_vec = a.nout % 4 == 0 && ((uintptr_t)part % 16) == 0;
        const hipError_t e = launch_prefill<kFmtMx, 64, 64, 2, 2, 3, 2>(as, st);
        if (e != hipSuccess) return e;
        const int64_t n = a.rows * a.nout;
        hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, pl.S, a.rows,
                           a.nout, a.y, a.ydt, a.ldy);
        return hipGetLastError();
    }
    if (pl.kernel >= 1) return launch_prefill<kFmtMx, 64, 64, 2, 2, 3, 2>(a, st);
    const int fm = a.rows <= 16 ? 1 : a.rows <= 32 ? 2 : a.rows <= 48 ? 3 : 4;
    if (fm == 1) return launch_small<1>(a, st);
    if (fm == 2) return launch_small<2>(a, st);
    if (fm == 3) return launch_small<3>(a, st);
    return launch_small<4>(a, st);
}

// SwiGLU-epilogue products (MXFP4): the tile shapes of launch_linear_mx whose
// waves hold gate/up fragment pairs, at any row count (no few-row kernels).
// Launches of at least two rounds of 128x256 tiles at two workgroups per CU
// take that shape (two stages): one workgroup's SwiGLU epilogue, about 4000
// vector instructions per wave, overlaps the other's matrix work (Llama
// gate_up 2048 x 28672 x 4096 on MI355X: 2% faster than 256x256 tiles with
// the column split).
template <int EPI>
static hipError_t launch_mx_swiglu(const LinearArgs &a, hipStream_t st) {
    if (a.offsets)
        return launch_prefill<kFmtMx, 128, 256, 2, 2, 2, 2, 0, 1, true, EPI>(a, st, 0, -1, a.E >= 16);
    const int64_t cus = device_cus();
    if (((a.rows + 127) / 128) * ((a.nout + 255) / 256) >= 2 * 2 * cus)
        return launch_prefill<kFmtMx, 128, 256, 2, 2, 2, 2, 0, 1, false, EPI>(a, st);
    double t_one = 0.0;
    const int one = best_shape(a.rows, a.nout, cus, &t_one, true);
    const int64_t mt = (a.rows + 255) / 256;
    const int64_t full_rounds = (mt * ((a.nout + 255) / 256)) / cus;
    const int64_t n_split = (full_rounds * cus / mt) * 256;
    if (full_rounds >= 1 && n_split > 0 && n_split < a.nout) {
        double t_rem = 0.0;
        const int rem = best_shape(a.rows, a.nout - n_split, cus, &t_rem, true);
        const double t_main = (double)((mt * (n_split / 256) + cus - 1) / cus) * 256 * 256;
        if (t_main + t_rem < 0.97 * t_one) {
            const hipError_t e = launch_mx_shape<EPI>(0, a, st, 0, n_split);
            if (e != hipSuccess) return e;
            return launch_mx_shape<EPI>(rem, a, st, n_split, a.nout);
        }
    }
    return launch_mx_shape<EPI>(one, a, st, 0, a.nout);
}

hipError_t launch_linear_swiglu(const LinearArgs &a, hipStream_t st) {
    if (a.p_m == 1) return launch_mx_swiglu<1>(a, st);
    if (a.p_m == 2) return launch_mx_swiglu<2>(a, st);
    return launch_mx_swiglu<4>(a, st);
}

static hipError_t launch_linear_mx(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st) {
    if (a.offsets == nullptr && a.rows <= 64) return launch_linear_mx_few_rows(a, ws, ws_bytes, st);
    // grouped expert products: 128x256 tiles, two stages, two workgroups per CU
    // (measured on MI355X on the Qwen3-30B-A3B expert shapes: 5% faster than
    // one workgroup with three stages at K = 2048, 11% at K = 768, where one
    // workgroup's output stores overlap the other's MFMAs)
    if (a.offsets) return launch_prefill<kFmtMx, 128, 256, 2, 2, 2, 2, 0, 1, true>(a, st, 0, -1, a.E >= 16);
    const int64_t cus = device_cus();
    double t_one = 0.0;
    const int one = best_shape(a.rows, a.nout, cus, &t_one);
    const int64_t mt = (a.rows + 255) / 256;
    const int64_t full_rounds = (mt * ((a.nout + 255) / 256)) / cus;
    const int64_t n_split = (full_rounds * cus / mt) * 256;
    if (full_rounds >= 1 && n_split > 0 && n_split < a.nout) {
        double t_rem = 0.0;
        const int rem = best_shape(a.rows, a.nout - n_split, cus, &t_rem);
        const double t_main = (double)((mt * (n_split / 256) + cus - 1) / cus) * 256 * 256;
        if (t_main + t_rem < 0.97 * t_one) {  // a second launch costs a little
            const hipError_t e = launch_mx_shape(0, a, st, 0, n_split);
            if (e != hipSuccess) return e;
            return launch_mx_shape(rem, a, st, n_split, a.nout);
        }
    }
    return launch_mx_shape(one, a, st, 0, a.nout);
}

// NVFP4 (f16 MFMA on fragments dequantized in registers): 128x128 tiles
// with two workgroups per CU (one workgroup's dequantization overlaps the
// other's MFMAs), or 256x256 tiles of four waves with 128x128 per wave
// (each dequantized fragment feeds four MFMAs instead of two: measured on
// MI355X 10-18% faster once there are enough tiles), whichever takes fewer
// rounds of tiles, weighted by the measured cost per output element
// (1.17 : 1); when 256x256 tiles fill some rounds and leave a partial one,
// the columns of the full rounds run as 256x256 tiles and the rest in a
// second launch of 64x128 tiles at three workgroups per CU, which spreads
// those few columns over every CU (Qwen2.5-7B qkv, 4096 x 4608 x 3584, on
// MI355X: 214 -> 196 us against 128x128 tiles at two per CU; 128x64 tiles
// 206-208).  A third shape, 256x224 tiles of four waves stacked along the
// rows (64x224 per wave), fills a round exactly where the output width is a
// multiple of 224 but not of 256 (Qwen2.5-7B o_proj and down, 4096 x 3584:
// 256 tiles instead of 224 of 256x256; measured 5% and 4% faster, a cost
// per output element of 1.085 against 256x256 tiles).  Grouped expert
// products use 128x256 tiles.  NVFP4_SP24 (backbone on the 2:4 sparse f16
// MFMA) uses the same shapes.
static double nv_cost128(int64_t rows, int64_t cols, int64_t cus) {
    const int64_t t = ((rows + 127) / 128) * ((cols + 127) / 128);
    return (double)((t + 2 * cus - 1) / (2 * cus)) * 2.0 * 128 * 128 * 1.17;
}
static double nv_cost256(int64_t rows, int64_t cols, int64_t cus) {
    const int64_t t = ((rows + 255) / 256) * ((cols + 255) / 256);
    return (double)((t + cus - 1) / cus) * 256.0 * 256;
}
static double nv_cost224(int64_t rows, int64_t cols, int64_t cus) {
    const int64_t t = ((rows + 255) / 256) * ((cols + 223) / 224);
    return (double)((t + cus - 1) / cus) * 256.0 * 224 * 1.085;
}

template <int FMT>
static hipError_t launch_linear_nv(const LinearArgs &a, hipStream_t st) {
    if (a.offsets) return launch_prefill<FMT, 128, 256, 2, 2, 3, 1, 4, 1, true>(a, st);
    const int64_t cus = device_cus();
    const double c128 = nv_cost128(a.rows, a.nout, cus), c256 = nv_cost256(a.rows, a.nout, cus);
    const double c224 = nv_cost224(a.rows, a.nout, cus);
    const double c_one = c128 < c256 ? (c128 < c224 ? c128 : c224) : (c256 < c224 ? c256 : c224);
    const int64_t mt = (a.rows + 255) / 256;
    const int64_t full_rounds = (mt * ((a.nout + 255) / 256)) / cus;
    const int64_t n_split = (full_rounds * cus / mt) * 256;
    if (full_rounds >= 1 && n_split > 0 && n_split < a.nout) {
        const double split = nv_cost256(a.rows, n_split, cus) + nv_cost128(a.rows, a.nout - n_split, cus);
        if (split < 0.97 * c_one) {  // a second launch costs a little
            const hipError_t e = launch_prefill<FMT, 256, 256, 2, 2, 2, 1, 0, 1>(a, st, 0, n_split);
            if (e != hipSuccess) return e;
            return launch_prefill<FMT, 64, 128, 2, 2, 2, 3, 0, 1>(a, st, n_split, a.nout);
        }
    }
    if (c224 == c_one && c224 < c256) return launch_prefill<FMT, 256, 224, 4, 1, 2, 1, 0, 1>(a, st);
    if (c256 < c128) return launch_prefill<FMT, 256, 256, 2, 2, 2, 1, 0, 1>(a, st);
    return launch_prefill<FMT, 128, 128, 2, 2, 2, 2, 0, 1>(a, st);
}

hipError_t launch_linear(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st) {
    if (a.fmt == kFmtMx) return launch_linear_mx(a, ws, ws_bytes, st);
    if (a.fmt == kFmtNvSp) return launch_linear_nv<kFmtNvSp>(a, st);
    return launch_linear_nv<kFmtNv>(a, st);
}

size_t linear_workspace_bytes(int64_t rows, int64_t K, int64_t nout, int64_t E, int fmt) {
    // partial products of a K-split few-row MXFP4 product (dense weight only)
    if (fmt != kFmtMx || E != 1 || rows <= 0 || rows > 64 || nout <= 0 || K <= 0 || K % 128 != 0) return 0;
    return few_rows_workspace(rows, K, nout);
}

}  // namespace sharq
