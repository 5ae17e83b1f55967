// Fused SharQ preparation kernels for gfx950.
//
// Source: SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference, Abstract.
// One operator normalizes a row, picks the N:M mask from the row's own
// magnitudes, quantizes the masked backbone to FP4, subtracts the
// dequantized backbone to get the dense residual and quantizes that too.
//
// Work decomposition: one wavefront per row task.  Lane l of a wave owns the
// eight consecutive elements [(c*64 + l)*8, +8) of chunk c of the row, so
// every global load is one coalesced 128-bit word per lane (1 KiB per wave),
// an N:M group with M <= 8 sits inside one lane, an MXFP4 block (32) spans
// the four lanes of a DPP quad and an NVFP4 block (16) a lane pair.  The row
// is read from HBM exactly once; everything else happens in registers.
//
//   MX + norm, K <= 8192:  a workgroup of two (K <= 2048) or four waves per
//                          row; the row stays in registers across the FP64
//                          norm reduction (whose per-wave partials meet in
//                          LDS) and the quantization pass, whose stores are
//                          buffer stores at scalar + per-lane-constant
//                          offsets;
//   MX + norm, larger K:   one wave per row, the quantization pass re-reads
//                          the row (L2 hit);
//   no norm:               tasks are (row, group of chunks), fully parallel;
//   NVFP4:                 a pre-pass writes per-row norm statistics and
//                          amax, a one-block kernel reduces the tensor scale,
//                          then the main pass streams (row, chunk-group) tasks.
#include <mutex>

#include "device_util.h"
#include "kernels.h"

namespace sharq {

constexpr int kPrepWaves = 4;        // waves per workgroup
constexpr int kChunk = 512;          // elements per wave-wide 128-bit load
constexpr int kStreamChunks = 1;     // chunks per task when rows are split (measured: 1 beats 2, 4 and 8)

struct RowStats {  // per-row statistics written by the NVFP4 pre-pass
    float r, mu, amax, pad;
};

// ---------------------------------------------------------------- selection
// (select_in_lane, select_2of4: device_util.h)

// M = 16: a group spans the lane and its quad neighbour (lane ^ 1); the lower
// lane of the pair holds group elements 0..7.
__device__ __forceinline__ uint32_t select_m16(const float v[8], int n, int lane) {
    uint32_t key[8], other[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        key[i] = __float_as_uint(v[i]) & 0x7FFFFFFFu;
        other[i] = dpp_u32<kDppQuadXor1>(key[i]);
    }
    const bool low = (lane & 1) == 0;
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if (j != i) rank += (j < i ? key[j] >= key[i] : key[j] > key[i]) ? 1 : 0;
            // partner elements come before ours when we are the upper lane
            rank += (low ? other[j] > key[i] : other[j] >= key[i]) ? 1 : 0;
        }
        keep |= (rank < n ? 1u : 0u) << i;
    }
    return keep;
}

// FAST24: 1 = the 2:4 fast path, 0 = runtime N with M-wide groups.  keep[i]
// is element i's flag (as a lane predicate).
template <int M, int FAST24>
__device__ __forceinline__ void select8(const float v[8], int n, int lane, bool keep[8]) {
    if constexpr (FAST24) {
        uint64_t km[8];
        select_2of4(v, km);
#pragma unroll
        for (int i = 0; i < 8; i++) keep[i] = __builtin_amdgcn_inverse_ballot_w64(km[i]);
    } else {
        uint32_t k;
        if constexpr (M == 16) k = select_m16(v, n, lane);
        else k = select_in_lane<M>(v, n);
#pragma unroll
        for (int i = 0; i < 8; i++) keep[i] = (k >> i) & 1u;
    }
}

// ---------------------------------------------------------------- block quantizers
// MXFP4: 32-element block across a quad.  Writes packed codes of the lane's
// eight elements, the dequantized values (if DEQ), and returns the E8M0 byte.
// The conversions take the block exponent as their scale operand, i.e. they
// round v * 2^-E and decode to code * 2^E, both exactly.
template <bool DEQ>
__device__ __forceinline__ uint32_t quant_mx8(const float s[8], uint32_t &codes, float deq[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(s[i]));
    const int E = mx_shared_exp(quad_max_nonneg(m));
    const float scale = e8m0_operand(E);
    codes = e2m1_cvt8(s, scale);
    if constexpr (DEQ) e2m1_dec8(codes, scale, deq);
    return (uint32_t)(E + 127);
}

// NVFP4: 16-element block across a lane pair, tensor scale G, rG6 = the
// double reciprocal of fl32(6G).  The two quotients the format defines,
// fl32(amax / fl32(6G)) and fl32(v / D), are formed as float(double(x) * r)
// with r the double reciprocal of the float divisor.  The quotient of two
// floats is never closer than 2^-49 (relative) to a midpoint M between
// adjacent floats: v = M*D would make the 24-bit significand of v a
// multiple of M's odd 25-bit one, and otherwise v and M*D differ by at least
// one unit of their common bit grid.  The double product is within 2^-52 of
// the quotient (plus 2^-79 from the reciprocal below), so both round to the
// same float.  (Quotients below the normal range can part at an exact tie
// of the subnormal grid; they lie far below the smallest E2M1 step and the
// smallest E4M3 scale and encode as zero either way.)  A zero divisor gives
// the same infinities and NaNs as the division.
//
// The element reciprocal 1/D is rcp_f64_refined (the hardware reciprocal
// after two Newton steps, within the final rounding plus 2^-79 of 1/D).  A
// block whose scale code is 0 (D = 0) takes r = 0: every quotient is then
// +-0, which the E2M1 conversion encodes as the canonical zero code.

__device__ __forceinline__ uint32_t quant_nv8(const float s[8], float G, double rG6, uint32_t &codes,
                                              float deq[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(s[i]));
    m = pair_max_nonneg(m);
    const uint32_t sb = e4m3_encode_sat((float)((double)m * rG6));
    const float D = __fmul_rn(e4m3_value(sb), G);
    const double rD = sb != 0u ? rcp_f64_refined((double)D) : 0.0;
    float u[8], q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) u[i] = (float)((double)s[i] * rD);
    codes = e2m1_cvt8(u, 1.0f);
    e2m1_dec8(codes, 1.0f, q);
#pragma unroll
    for (int i = 0; i < 8; i++) deq[i] = __fmul_rn(q[i], D);
    return sb;
}

// ---------------------------------------------------------------- normalization
template <int NORM>
__device__ __forceinline__ void normalize8(float v[8], const float g[8], const float b[8], float r,
                                           float mu) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        if constexpr (NORM == kNormRms) {
            v[i] = __fmul_rn(__fmul_rn(v[i], r), g[i]);
        } else if constexpr (NORM == kNormLayer) {
            v[i] = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(v[i], mu), r), g[i]), b[i]);
        }
    }
}

template <bool BF16, bool HAS>
__device__ __forceinline__ void load_param8(const uint16_t *p, int64_t e0, float out[8], float dflt) {
    if (HAS && p != nullptr) {
        unpack8<BF16>(*reinterpret_cast<const uint4 *>(p + e0), out);
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) out[i] = dflt;
    }
}

// Raw 128-bit word of a per-column parameter (gamma, beta), loaded early so
// its latency overlaps the row's own loads; absent parameters read as the
// bit pattern of dflt in every element.
template <bool HAS>
__device__ __forceinline__ uint4 param_raw(const uint16_t *p, int64_t e0, uint32_t dflt_pair) {
    if (HAS && p != nullptr) return *reinterpret_cast<const uint4 *>(p + e0);
    return make_uint4(dflt_pair, dflt_pair, dflt_pair, dflt_pair);
}

// ---------------------------------------------------------------- per-chunk body
// Normalized values v of one lane -> mask byte, backbone and residual codes
// and scales, stored at element offset e0 of row `row`.
//
// Store addressing (K % 128 == 0 and every output array below 4 GiB, the
// usual case): buffer stores whose byte offset is a wave-uniform part (row
// and chunk, in a scalar register) plus a per-lane constant, so no per-lane
// address arithmetic runs per store.  A wave-wide chunk (512 elements, chunk
// index ch along K) starts on a K-tile boundary: lane l holds elements
// (l%16)*8 .. +7 of K tile 4ch + l/16.  Its code dword lies at
// ch*T*256 + row*64 + [q*T*64 + (l%16)*4], q = l/16, the bracket being the
// per-lane constant.  The tile's block-scale bytes of the row (4 MX, 8
// NVFP4) are gathered by DPP into dwords and stored by one lane per dword.
// Other shapes take per-lane 64-bit K-tiled offsets.
struct LaneOff {
    uint32_t co;  // code dword
    uint32_t so;  // scale dword (lanes that store one)
    // NVFP4_SP24 backbone (lanes that store one, else out of range): chunk
    // dword, index dword, scale dword
    uint32_t spc, spi, sps;
};

// NVFP4_SP24 backbone of one K tile and row (48 bytes, lane w = lane % 16
// holds elements 8w..8w+7): lanes 8..15 store chunk c = 4p + 2h + u of the
// kept codes (p = bit 2 of w, h = bit 0, u = bit 1; the first four codes from
// lane w-8, the last four their own) at byte 4c; lanes 10, 11, 14 and 15
// store the index dword of (p, h) at byte 32 + 4(2p + h); lanes 10 and 14
// store the tile's scale dwords (blocks 0, 1, 4, 5 and 2, 3, 6, 7).
template <int FMT>
__device__ __forceinline__ LaneOff lane_offsets(const PrepArgs &a, int lane) {
    constexpr uint32_t SPT = FMT == kFmtMx ? 4 : 8;  // scale bytes per row per K tile
    const uint32_t q = (uint32_t)lane >> 4, w = (uint32_t)lane & 15u;
    LaneOff o{q * (uint32_t)(a.T * (kTileK / 2)) + w * 4u,
              q * (uint32_t)a.T * SPT + (FMT == kFmtMx ? 0u : (w >= 8u ? 4u : 0u)), kOutOfRange, kOutOfRange,
              kOutOfRange};
    if (FMT == kFmtNv && a.sp) {
        const uint32_t tile = q * (uint32_t)a.T * kSpRowBytes, p = (w >> 2) & 1u, h = w & 1u, u = (w >> 1) & 1u;
        if (w >= 8u) o.spc = tile + 4u * (4u * p + 2u * h + u);
        if (w >= 8u && u == 1u) o.spi = tile + 32u + 4u * (2u * p + h);
        if (w == 10u || w == 14u) o.sps = q * (uint32_t)a.T * SPT + (w == 10u ? 0u : 4u);
    }
    return o;
}

// Scale bytes of a lane's block, gathered so that one lane per dword holds
// the dword of the K tile's scales of this row: MX (four blocks of four
// lanes) in lanes 16q+12..15; NVFP4 (eight blocks of two lanes) bytes 0-3 in
// lanes 16q+6, 7 and bytes 4-7 in lanes 16q+14, 15.
template <int FMT>
__device__ __forceinline__ uint32_t gather_scales(uint32_t sb, int lane) {
    constexpr int kRowShr = 0x110;  // DPP row_shr:n = 0x110 + n (within rows of 16 lanes)
    if constexpr (FMT == kFmtMx) {
        uint32_t v = sb << (8 * ((lane >> 2) & 3));
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 4, 0xF, 0xF, true);
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 8, 0xF, 0xF, true);
        return v;
    } else {
        uint32_t v = sb << (8 * ((lane >> 1) & 3));
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 2, 0xF, 0xF, true);
        v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 4, 0xF, 0xF, true);
        return v;
    }
}

// The backbone's scale bytes in the NVFP4_SP24 order: the dword of blocks
// 0, 1, 4, 5 of the K tile in lane 16q+10, that of blocks 2, 3, 6, 7 in lane
// 16q+14 (block b is held by lanes 2b and 2b+1).
__device__ __forceinline__ uint32_t gather_scales_sp(uint32_t sb, int lane) {
    constexpr int kRowShr = 0x110;
    const int w = lane & 15;
    uint32_t v = sb << (8 * (((w >> 1) & 1) | (((w >> 3) & 1) << 1)));
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 2, 0xF, 0xF, true);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr + 8, 0xF, 0xF, true);
    return v;
}

// 2:4 compression of a lane's eight backbone codes (exactly two kept per
// group of four): the kept codes of each group in ascending position (four
// codes, 16 bits) and their positions (2 bits each, 8 bits).
__device__ __forceinline__ void compress24(uint32_t codes, const bool kp[8], uint32_t &cc, uint32_t &ix) {
    cc = 0;
    ix = 0;
#pragma unroll
    for (int g = 0; g < 2; g++) {
        const uint32_t p0 = kp[4 * g] ? 0u : (kp[4 * g + 1] ? 1u : 2u);
        const uint32_t p1 = kp[4 * g + 3] ? 3u : (kp[4 * g + 2] ? 2u : 1u);
        const uint32_t c0 = (codes >> (16 * g + 4 * p0)) & 0xFu, c1 = (codes >> (16 * g + 4 * p1)) & 0xFu;
        cc |= (c0 | (c1 << 4)) << (8 * g);
        ix |= (p0 | (p1 << 2)) << (4 * g);
    }
}

template <int FMT>
__device__ __forceinline__ bool scale_store_lane(int lane) {
    return FMT == kFmtMx ? (lane & 15) == 12 : (lane & 7) == 6;
}

// Decompose eight consecutive normalized values (elements 8*lane .. +7 of
// chunk ch of `row`; row and ch wave-uniform) and store their share of the
// mask, codes and scales.  OFF32 (K % 128 == 0, every output array below
// 2 GiB): buffer stores at scalar + per-lane-constant offsets, the same
// instructions on every lane and call (lanes that store no scale dword, and
// every lane when there is no mask, write out of range, which the buffer
// unit drops), so the compiler can count outstanding memory operations
// exactly and a row loop never waits for its stores.  Otherwise per-lane
// 64-bit K-tiled offsets.
template <int FMT, int M, int FAST24, bool OFF32, bool SP = false>
__device__ __forceinline__ void decompose_store(const PrepArgs &a, int64_t row, int64_t ch, int lane, LaneOff lo,
                                                const float v[8], float G, double rG6) {
    static_assert(!SP || (FMT == kFmtNv && M == 4 && FAST24 && OFF32), "the compressed backbone is NVFP4 2:4");
    bool kp[8];
    select8<M, FAST24>(v, a.n, lane, kp);
    float S[8], dq[8], R[8];
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        S[i] = kp[i] ? v[i] : 0.0f;
        keep |= kp[i] ? (1u << i) : 0u;
    }
    uint32_t bc, rc, bs, rs;
    if constexpr (FMT == kFmtMx) bs = quant_mx8<true>(S, bc, dq);
    else bs = quant_nv8(S, G, rG6, bc, dq);
#pragma unroll
    for (int i = 0; i < 8; i++) R[i] = __fsub_rn(v[i], dq[i]);
    float unused[8];
    if constexpr (FMT == kFmtMx) rs = quant_mx8<false>(R, rc, unused);
    else rs = quant_nv8(R, G, rG6, rc, unused);

    const int64_t K = a.K;
    constexpr int LPB = FMT == kFmtMx ? 4 : 2;  // lanes per scale block
    constexpr int B = FMT == kFmtMx ? 32 : 16;
    if constexpr (OFF32) {
        constexpr uint32_t SPT = FMT == kFmtMx ? 4 : 8;
        const uint32_t T = (uint32_t)a.T, r32 = (uint32_t)row, c32 = (uint32_t)ch;
        const int soc = __builtin_amdgcn_readfirstlane((int)(c32 * T * (kChunk / 2) + r32 * (kTileK / 2)));
        const int sos = __builtin_amdgcn_readfirstlane((int)(c32 * T * (4 * SPT) + r32 * SPT));
        const int som = __builtin_amdgcn_readfirstlane((int)(r32 * (uint32_t)(K / 8) + c32 * (kChunk / 8)));
        const uint32_t ncodes = T * (uint32_t)(K / 2), nsc = T * (uint32_t)(K / B);
        const uint32_t nmask = a.mask ? T * (uint32_t)(K / 8) : 0u;  // no mask: every store dropped
        const uint32_t sv = scale_store_lane<FMT>(lane) ? lo.so : kOutOfRange;
        if constexpr (SP) {
            constexpr int kRowShr = 0x110;
            uint32_t cc, ix;
            compress24(bc, kp, cc, ix);
            const uint32_t chunk = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cc, kRowShr + 8, 0xF, 0xF, true) |
                                   (cc << 16);
            const uint32_t ix16 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ix, kRowShr + 8, 0xF, 0xF, true) |
                                  (ix << 8);
            const uint32_t ix32 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ix16, kRowShr + 2, 0xF, 0xF, true) |
                                  (ix16 << 16);
            const int sob = __builtin_amdgcn_readfirstlane(
                (int)(c32 * T * (4 * kSpRowBytes) + r32 * kSpRowBytes));
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.b_codes, T * (uint32_t)(K / kTileK) * kSpRowBytes);
            __builtin_amdgcn_raw_buffer_store_b32(chunk, rb, (int)lo.spc, sob, 0);
            __builtin_amdgcn_raw_buffer_store_b32(ix32, rb, (int)lo.spi, sob, 0);
            __builtin_amdgcn_raw_buffer_store_b32(gather_scales_sp(bs, lane), make_rsrc(a.b_scales, nsc), (int)lo.sps,
                                                  sos, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(bc, make_rsrc(a.b_codes, ncodes), (int)lo.co, soc, 0);
            __builtin_amdgcn_raw_buffer_store_b32(gather_scales<FMT>(bs, lane), make_rsrc(a.b_scales, nsc), (int)sv,
                                                  sos, 0);
        }
        __builtin_amdgcn_raw_buffer_store_b32(rc, make_rsrc(a.r_codes, ncodes), (int)lo.co, soc, 0);
        __builtin_amdgcn_raw_buffer_store_b32(gather_scales<FMT>(rs, lane), make_rsrc(a.r_scales, nsc), (int)sv, sos, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)keep, make_rsrc(a.mask, nmask), lane, som, 0);
    } else {
        if (a.mask) (a.mask + row * (K / 8) + ch * (kChunk / 8))[lane] = (uint8_t)keep;
        const int64_t e0 = ch * kChunk + lane * 8;
        const int64_t co = ktile_offset<2>(row, e0, a.T, K);
        const int64_t so = ktile_offset<B>(row, e0, a.T, K);
        *reinterpret_cast<uint32_t *>(a.b_codes + co) = bc;
        *reinterpret_cast<uint32_t *>(a.r_codes + co) = rc;
        if ((lane % LPB) == 0) {
            a.b_scales[so] = (uint8_t)bs;
            a.r_scales[so] = (uint8_t)rs;
        }
    }
}

// Either store path, chosen per launch.
template <int FMT, int M, int FAST24>
__device__ __forceinline__ void decompose_any(const PrepArgs &a, int64_t row, int64_t ch, int lane, LaneOff lo,
                                              const float v[8], float G, double rG6) {
    if constexpr (FMT == kFmtNv && M == 4 && FAST24) {
        if (a.sp) {
            decompose_store<FMT, M, FAST24, true, true>(a, row, ch, lane, lo, v, G, rG6);
            return;
        }
    }
    if (a.off32)
        decompose_store<FMT, M, FAST24, true>(a, row, ch, lane, lo, v, G, rG6);
    else
        decompose_store<FMT, M, FAST24, false>(a, row, ch, lane, lo, v, G, rG6);
}

// ---------------------------------------------------------------- MX, norm, one row per workgroup
// A workgroup of NWG waves handles one row; wave w owns chunks w, w+NWG, ...
// of it (at most CPW of them, held in registers from one batch of loads).
// Each wave reduces its FP64 partial sums, the NWG partials meet in LDS and
// every wave adds them in the same fixed order, so all waves derive the same
// r (and mu).  Row loads are buffer loads from the row's scalar base, so no
// per-lane address arithmetic.
template <bool BF16, int NORM, int M, int FAST24, int CPW, int NWG, bool FULL>
struct NormRows {
    static constexpr uint32_t kOnePair = BF16 ? 0x3F803F80u : 0x3C003C00u;  // 1.0, 1.0

    // Row `row`'s words (chunks past the row's end read as zeros).
    static __device__ __forceinline__ void load_row(const PrepArgs &a, int64_t row, int wave, int lane,
                                                    const bool (&in)[CPW], uint4 (&raw)[CPW]) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(a.x + row * a.ldx, (uint32_t)(a.K * 2));
#pragma unroll
        for (int j = 0; j < CPW; j++) {
            const uint32_t off = (uint32_t)(((wave + NWG * j) * kWave + lane) * 16);
            raw[j] = bload128(r, in[j] ? off : kOutOfRange);
        }
    }

    // Norm statistics of one row (every wave of the workgroup gets the same),
    // then the decomposition of the wave's chunks.
    static __device__ __forceinline__ void row(const PrepArgs &a, int64_t row, int slot, int wave, int lane,
                                               LaneOff lo, const bool (&in)[CPW], const uint4 (&raw)[CPW],
                                               const float (&gf)[CPW][8], const float (&bf)[CPW][8],
                                               double (&part)[2][2][NWG]) {
        const int64_t K = a.K;
        float xf[CPW][8];
#pragma unroll
        for (int j = 0; j < CPW; j++) unpack8<BF16>(raw[j], xf[j]);  // out-of-range words are 0
        double s1 = 0.0, s1b = 0.0;
#pragma unroll
        for (int j = 0; j < CPW; j++) {
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                if constexpr (NORM == kNormRms) {
                    s1 = __fma_rn((double)xf[j][i], (double)xf[j][i], s1);  // x*x exact in double
                    s1b = __fma_rn((double)xf[j][i + 1], (double)xf[j][i + 1], s1b);
                } else {
                    s1 += (double)xf[j][i];
                    s1b += (double)xf[j][i + 1];
                }
            }
        }
        s1 = wave_sum_f64(s1 + s1b);
        if (lane == 0) part[slot][0][wave] = s1;
        __syncthreads();
        s1 = part[slot][0][0];
#pragma unroll
        for (int w = 1; w < NWG; w++) s1 += part[slot][0][w];
        float r, mu = 0.0f;
        if constexpr (NORM == kNormRms) {
            r = (float)(1.0 / sqrt(s1 / (double)K + (double)a.eps));
        } else {
            const double mud = s1 / (double)K;
            double s2 = 0.0;
#pragma unroll
            for (int j = 0; j < CPW; j++) {
                if (in[j]) {
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const double d = (double)xf[j][i] - mud;
                        s2 += d * d;  // d*d is rounded on its own, as in the definition
                    }
                }
            }
            s2 = wave_sum_f64(s2);
            if (lane == 0) part[slot][1][wave] = s2;
            __syncthreads();
            s2 = part[slot][1][0];
#pragma unroll
            for (int w = 1; w < NWG; w++) s2 += part[slot][1][w];
            mu = (float)mud;
            r = (float)(1.0 / sqrt(s2 / (double)K + (double)a.eps));
        }
#pragma unroll
        for (int j = 0; j < CPW; j++) {
            if (in[j]) {
                normalize8<NORM>(xf[j], gf[j], bf[j], r, mu);
                decompose_store<kFmtMx, M, FAST24, true>(a, row, wave + NWG * j, lane, lo, xf[j], 1.0f, 0.0);
            }
        }
    }
};

// One row per workgroup, FULL: K == CPW * NWG * 512 (every chunk of every
// wave is in the row).  Launched only with the 32-bit store offsets
// (K % 128 == 0, outputs below 2 GiB).  One row per workgroup beat two or
// four consecutive rows with the next row prefetched (measured on MI355X at
// 2048 and 4096 rows of 4096): with no second register buffer 8 waves fit
// on a SIMD, so every row of such a launch is resident and loading at once.
template <bool BF16, int NORM, int M, int FAST24, int CPW, int NWG, bool FULL>
__global__ __launch_bounds__(NWG * kWave) void k_prep_mx_rows(PrepArgs a) {
    using R = NormRows<BF16, NORM, M, FAST24, CPW, NWG, FULL>;
    __shared__ double part[2][2][NWG];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const LaneOff lo = lane_offsets<kFmtMx>(a, lane);
    const int64_t row = xcd_block(blockIdx.x, gridDim.x);
    if (row >= a.T) return;
    const int64_t K = a.K;

    bool in[CPW];
    float gf[CPW][8], bf[CPW][8];
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int64_t e0 = ((int64_t)(wave + NWG * j) * kWave + lane) * 8;
        in[j] = FULL || e0 < K;
        const uint4 g = in[j] ? param_raw<true>(a.gamma, e0, R::kOnePair) : make_uint4(0, 0, 0, 0);
        const uint4 b = in[j] ? param_raw<NORM == kNormLayer>(a.beta, e0, 0u) : make_uint4(0, 0, 0, 0);
        unpack8<BF16>(g, gf[j]);
        unpack8<BF16>(b, bf[j]);
    }
    uint4 x[CPW];
    R::load_row(a, row, wave, lane, in, x);
    R::row(a, row, 0, wave, lane, lo, in, x, gf, bf, part);
}

// ---------------------------------------------------------------- MX, norm, two reads
template <bool BF16, int NORM, int M, int FAST24>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_prep_mx_2pass(PrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = xcd_block(blockIdx.x, gridDim.x) * kPrepWaves + wave;
    if (row >= a.T) return;
    const uint16_t *xr = a.x + row * a.ldx;
    const int64_t K = a.K;
    float v[8];
    double s1 = 0.0;
    for (int64_t e0 = (int64_t)lane * 8; e0 < K; e0 += kChunk) {
        unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if constexpr (NORM == kNormRms) s1 = __fma_rn((double)v[i], (double)v[i], s1);  // x*x exact in double
            else s1 += (double)v[i];
        }
    }
    s1 = wave_sum_f64(s1);
    float r, mu = 0.0f;
    if constexpr (NORM == kNormRms) {
        r = (float)(1.0 / sqrt(s1 / (double)K + (double)a.eps));
    } else {
        const double mud = s1 / (double)K;
        double s2 = 0.0;
        for (int64_t e0 = (int64_t)lane * 8; e0 < K; e0 += kChunk) {
            unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const double d = (double)v[i] - mud;
                s2 += d * d;  // d*d is rounded on its own, as in the definition
            }
        }
        s2 = wave_sum_f64(s2);
        mu = (float)mud;
        r = (float)(1.0 / sqrt(s2 / (double)K + (double)a.eps));
    }
    const LaneOff lo = lane_offsets<kFmtMx>(a, lane);
    for (int64_t ch = 0; ch * kChunk < K; ch++) {
        const int64_t e0 = ch * kChunk + lane * 8;
        if (e0 < K) {
            float g[8], b[8];
            load_param8<BF16, true>(a.gamma, e0, g, 1.0f);
            load_param8<BF16, NORM == kNormLayer>(a.beta, e0, b, 0.0f);
            unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
            normalize8<NORM>(v, g, b, r, mu);
            decompose_any<kFmtMx, M, FAST24>(a, row, ch, lane, lo, v, 1.0f, 0.0);
        }
    }
}

// ---------------------------------------------------------------- streaming tasks
// Row-split tasks: (row, kStreamChunks chunks).  Normalization statistics
// come from the NVFP4 pre-pass (stats != nullptr) or there is no norm.  One
// task per wave.
template <bool BF16, int NORM>
__device__ __forceinline__ void stream_load(const PrepArgs &a, int64_t task, int64_t tpr, int lane,
                                            uint4 raw[kStreamChunks], uint4 graw[kStreamChunks],
                                            uint4 braw[kStreamChunks]) {
    constexpr uint32_t kOnePair = BF16 ? 0x3F803F80u : 0x3C003C00u;  // 1.0, 1.0
    const int64_t row = task / tpr;
    const int64_t c0 = (task - row * tpr) * kStreamChunks;
    const uint16_t *xr = a.x + row * a.ldx;
#pragma unroll
    for (int c = 0; c < kStreamChunks; c++) {
        const int64_t e0 = ((c0 + c) * kWave + lane) * 8;
        raw[c] = e0 < a.K ? *reinterpret_cast<const uint4 *>(xr + e0) : make_uint4(0, 0, 0, 0);
        if constexpr (NORM != kNormNone) {
            graw[c] = e0 < a.K ? param_raw<true>(a.gamma, e0, kOnePair) : make_uint4(0, 0, 0, 0);
            braw[c] = e0 < a.K ? param_raw<NORM == kNormLayer>(a.beta, e0, 0u) : make_uint4(0, 0, 0, 0);
        }
    }
}

template <bool BF16, int NORM, int FMT, int M, int FAST24, bool OFF32>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_prep_stream(PrepArgs a, const RowStats *stats) {
    const int lane = threadIdx.x & 63;
    const int64_t K = a.K;
    const int64_t tpr = (K + (int64_t)kChunk * kStreamChunks - 1) / ((int64_t)kChunk * kStreamChunks);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t task = xcd_block(blockIdx.x, gridDim.x) * kPrepWaves + wave;
    if (task >= a.T * tpr) return;
    const LaneOff lo = lane_offsets<FMT>(a, lane);
    float G = 1.0f;
    double rG6 = 0.0;  // 1 / fl32(6G), NVFP4 only
    if constexpr (FMT == kFmtNv) {
        G = *a.global_scale;
        rG6 = 1.0 / (double)__fmul_rn(6.0f, G);
    }
    uint4 raw[kStreamChunks], graw[kStreamChunks], braw[kStreamChunks];
    stream_load<BF16, NORM>(a, task, tpr, lane, raw, graw, braw);
    const int64_t row = task / tpr;
    const int64_t c0 = (task - row * tpr) * kStreamChunks;
    float r = 1.0f, mu = 0.0f;
    if constexpr (NORM != kNormNone) {
        r = stats[row].r;
        mu = stats[row].mu;
    }
#pragma unroll
    for (int c = 0; c < kStreamChunks; c++) {
        if ((c0 + c) * kChunk + lane * 8 < K) {
            float v[8];
            unpack8<BF16>(raw[c], v);
            if constexpr (NORM != kNormNone) {
                float g[8], b[8];
                unpack8<BF16>(graw[c], g);
                unpack8<BF16>(braw[c], b);
                normalize8<NORM>(v, g, b, r, mu);
            }
            if constexpr (FMT == kFmtNv && M == 4 && FAST24 && OFF32) {
                if (a.sp) {
                    decompose_store<FMT, M, FAST24, true, true>(a, row, c0 + c, lane, lo, v, G, rG6);
                    continue;
                }
            }
            decompose_store<FMT, M, FAST24, OFF32>(a, row, c0 + c, lane, lo, v, G, rG6);
        }
    }
}

// ---------------------------------------------------------------- SiLU(gate) * up source
// (exp32_fixed, silu_times, silu_times_n: device_util.h)

// Eight activations at element e0 of a row from its gate and up words.
__device__ __forceinline__ void swiglu8(const float *row, int64_t K, int64_t e0, float v[8]) {
    const float4 g0 = *reinterpret_cast<const float4 *>(row + e0);
    const float4 g1 = *reinterpret_cast<const float4 *>(row + e0 + 4);
    const float4 u0 = *reinterpret_cast<const float4 *>(row + K + e0);
    const float4 u1 = *reinterpret_cast<const float4 *>(row + K + e0 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    silu_times_n<8>(g, u, v);
}

// (row, kSwiChunks chunks) tasks, one per wave: one 512-element chunk per
// task (measured on MI355X at 2048 x 14336: 4% faster than two, 10% faster
// than four; more waves in flight hide the FP32 loads better).
constexpr int kSwiChunks = 1;

template <int FMT, int M, int FAST24>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_prep_swiglu(PrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = a.K;
    const int64_t tpr = (K + (int64_t)kChunk * kSwiChunks - 1) / ((int64_t)kChunk * kSwiChunks);
    const int64_t task = xcd_block(blockIdx.x, gridDim.x) * kPrepWaves + wave;
    const int64_t row = task / tpr;
    if (row >= a.T) return;
    const int64_t c0 = (task - row * tpr) * kSwiChunks;
    const float *gr = a.gu + row * a.ldgu;
    const LaneOff lo = lane_offsets<FMT>(a, lane);
    float G = 1.0f;
    double rG6 = 0.0;  // 1 / fl32(6G), NVFP4 only
    if constexpr (FMT == kFmtNv) {
        G = *a.global_scale;
        rG6 = 1.0 / (double)__fmul_rn(6.0f, G);
    }
#pragma unroll
    for (int c = 0; c < kSwiChunks; c++) {
        const int64_t e0 = (c0 + c) * kChunk + lane * 8;
        if (e0 < K) {
            float v[8];
            swiglu8(gr, K, e0, v);
            decompose_any<FMT, M, FAST24>(a, row, c0 + c, lane, lo, v, G, rG6);
        }
    }
}

// NVFP4: per-row amax of the activation (stats[row].amax; r = 1, mu = 0).
__global__ __launch_bounds__(kPrepWaves * kWave) void k_swiglu_rowstats(PrepArgs a, RowStats *stats) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kPrepWaves + (threadIdx.x >> 6);
    if (row >= a.T) return;
    const float *gr = a.gu + row * a.ldgu;
    float m = 0.0f, v[8];
    for (int64_t e0 = (int64_t)lane * 8; e0 < a.K; e0 += kChunk) {
        swiglu8(gr, a.K, e0, v);
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) stats[row] = RowStats{1.0f, 0.0f, m, 0.0f};
}

// ---------------------------------------------------------------- NVFP4 pre-pass
// Per row: norm statistics and amax of the normalized row, one row per
// workgroup of kPrepWaves waves with all of the row's words loaded at once
// (wave w owns chunks w, w+kPrepWaves, ..., at most CPW of them); the FP64
// partial sums and the partial maxima meet in LDS and are combined in a
// fixed order.  Rows longer than kPrepWaves*CPW chunks use k_nv_rowstats.
template <bool BF16, int NORM, int CPW>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_nv_rowstats_wg(PrepArgs a, RowStats *stats) {
    __shared__ double part[2][kPrepWaves];
    __shared__ float pmax[kPrepWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = xcd_block(blockIdx.x, gridDim.x);
    if (row >= a.T) return;
    const int64_t K = a.K;
    bool in[CPW];
    uint4 raw[CPW];
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int64_t e0 = ((int64_t)(wave + kPrepWaves * j) * kWave + lane) * 8;
        in[j] = e0 < K;
        raw[j] = in[j] ? *reinterpret_cast<const uint4 *>(a.x + row * a.ldx + e0) : make_uint4(0, 0, 0, 0);
    }
    float v[8];
    float r = 1.0f, mu = 0.0f;
    if constexpr (NORM != kNormNone) {
        double s1 = 0.0;
#pragma unroll
        for (int j = 0; j < CPW; j++) {
            unpack8<BF16>(raw[j], v);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if constexpr (NORM == kNormRms) s1 = __fma_rn((double)v[i], (double)v[i], s1);  // x*x exact in double
                else s1 += (double)v[i];
            }
        }
        s1 = wave_sum_f64(s1);
        if (lane == 0) part[0][wave] = s1;
        __syncthreads();
        s1 = part[0][0];
#pragma unroll
        for (int w = 1; w < kPrepWaves; w++) s1 += part[0][w];
        if constexpr (NORM == kNormRms) {
            r = (float)(1.0 / sqrt(s1 / (double)K + (double)a.eps));
        } else {
            const double mud = s1 / (double)K;
            double s2 = 0.0;
#pragma unroll
            for (int j = 0; j < CPW; j++) {
                if (in[j]) {
                    unpack8<BF16>(raw[j], v);
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const double d = (double)v[i] - mud;
                        s2 += d * d;  // d*d is rounded on its own, as in the definition
                    }
                }
            }
            s2 = wave_sum_f64(s2);
            if (lane == 0) part[1][wave] = s2;
            __syncthreads();
            s2 = part[1][0];
#pragma unroll
            for (int w = 1; w < kPrepWaves; w++) s2 += part[1][w];
            mu = (float)mud;
            r = (float)(1.0 / sqrt(s2 / (double)K + (double)a.eps));
        }
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        if (in[j]) {
            const int64_t e0 = ((int64_t)(wave + kPrepWaves * j) * kWave + lane) * 8;
            unpack8<BF16>(raw[j], v);
            if constexpr (NORM != kNormNone) {
                float g[8], b[8];
                load_param8<BF16, true>(a.gamma, e0, g, 1.0f);
                load_param8<BF16, NORM == kNormLayer>(a.beta, e0, b, 0.0f);
                normalize8<NORM>(v, g, b, r, mu);
            }
#pragma unroll
            for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) pmax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kPrepWaves; w++) m = fmaxf(m, pmax[w]);
        stats[row] = RowStats{r, mu, m, 0.0f};
    }
}

// Per row: norm statistics and amax of the normalized row, one row per wave
// looping over the row (any K; the row is read twice with a norm, three
// times with LayerNorm, the later reads mostly from cache).
template <bool BF16, int NORM>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_nv_rowstats(PrepArgs a, RowStats *stats) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kPrepWaves + (threadIdx.x >> 6);
    if (row >= a.T) return;
    const uint16_t *xr = a.x + row * a.ldx;
    const int64_t K = a.K;
    float v[8];
    float r = 1.0f, mu = 0.0f;
    if constexpr (NORM != kNormNone) {
        double s1 = 0.0;
        for (int64_t e0 = (int64_t)lane * 8; e0 < K; e0 += kChunk) {
            unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if constexpr (NORM == kNormRms) s1 = __fma_rn((double)v[i], (double)v[i], s1);  // x*x exact in double
                else s1 += (double)v[i];
            }
        }
        s1 = wave_sum_f64(s1);
        if constexpr (NORM == kNormRms) {
            r = (float)(1.0 / sqrt(s1 / (double)K + (double)a.eps));
        } else {
            const double mud = s1 / (double)K;
            double s2 = 0.0;
            for (int64_t e0 = (int64_t)lane * 8; e0 < K; e0 += kChunk) {
                unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const double d = (double)v[i] - mud;
                    s2 += d * d;  // d*d is rounded on its own, as in the definition
                }
            }
            s2 = wave_sum_f64(s2);
            mu = (float)mud;
            r = (float)(1.0 / sqrt(s2 / (double)K + (double)a.eps));
        }
    }
    float m = 0.0f;
    for (int64_t e0 = (int64_t)lane * 8; e0 < K; e0 += kChunk) {
        float g[8], b[8];
        unpack8<BF16>(*reinterpret_cast<const uint4 *>(xr + e0), v);
        if constexpr (NORM != kNormNone) {
            load_param8<BF16, true>(a.gamma, e0, g, 1.0f);
            load_param8<BF16, NORM == kNormLayer>(a.beta, e0, b, 0.0f);
            normalize8<NORM>(v, g, b, r, mu);
        }
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) stats[row] = RowStats{r, mu, m, 0.0f};
}

// Tensor scale G = fl32(amax / 2688), or 1 when that is not positive.
__global__ __launch_bounds__(1024) void k_nv_tensor_scale(const RowStats *stats, int64_t T, float *G) {
    __shared__ float part[1024 / kWave];
    // eight independent loads in flight per thread (max is exact in any order)
    constexpr int kU = 8;
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < T; i += kU * (int64_t)blockDim.x) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int64_t j = i + u * (int64_t)blockDim.x;
            v[u] = j < T ? stats[j].amax : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kU; u++) m = fmaxf(m, v[u]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int i = 0; i < (int)(blockDim.x / kWave); i++) t = fmaxf(t, part[i]);
        float g = __fdiv_rn(t, 2688.0f);
        *G = g > 0.0f ? g : 1.0f;
    }
}

__global__ void k_fill_f32(float *p, float v) { *p = v; }

// ---------------------------------------------------------------- launcher
// The rows kernel for NWG waves of CPW chunks each: full rows
// (K = CPW * NWG * 512) on the 2:4 path get the instantiation without bounds
// checks.
template <bool BF16, int NORM, int M, int FAST24, int CPW, int NWG>
static void launch_rows(const PrepArgs &a, bool full, hipStream_t st) {
    const dim3 grid((unsigned)round_up8(a.T)), blk(NWG * kWave);
    if (FAST24 && full)
        hipLaunchKernelGGL((k_prep_mx_rows<BF16, NORM, M, FAST24, CPW, NWG, true>), grid, blk, 0, st, a);
    else
        hipLaunchKernelGGL((k_prep_mx_rows<BF16, NORM, M, FAST24, CPW, NWG, false>), grid, blk, 0, st, a);
}

template <bool BF16, int NORM, int FMT, int M, int FAST24>
static hipError_t launch_prep_t(const PrepArgs &a, void *ws, hipStream_t st) {
    const dim3 blk(kPrepWaves * kWave);
    const int64_t K = a.K;
    if constexpr (FMT == kFmtMx && NORM != kNormNone) {
        constexpr int64_t kWg = (int64_t)kChunk * kPrepWaves;  // elements per chunk round of the workgroup
        if (!a.off32 || K > 4 * kWg) {
            const dim3 grid((unsigned)round_up8((a.T + kPrepWaves - 1) / kPrepWaves));
            hipLaunchKernelGGL((k_prep_mx_2pass<BF16, NORM, M, FAST24>), grid, blk, 0, st, a);
        } else if (K <= kWg) {
            // rows of up to 2048: two waves of two chunks (measured on MI355X
            // at 4096 x 2048: 10% faster than four waves of one chunk, as fast
            // as one wave of four)
            launch_rows<BF16, NORM, M, FAST24, 2, 2>(a, K == kWg, st);
        } else if (K <= 2 * kWg) {
            // rows of up to 4096: four waves of two chunks (two waves of four
            // were 5% slower at 2048 x 4096, eight waves of one 12% slower);
            // batches of at most 64 rows, one round of latency-bound
            // workgroups, take eight waves of one chunk (decode of 1, 8 and
            // 64 tokens at 4096: 5% faster, two waves of four 25% slower)
            if (a.T <= 64)
                launch_rows<BF16, NORM, M, FAST24, 1, 2 * kPrepWaves>(a, K == 2 * kWg, st);
            else
                launch_rows<BF16, NORM, M, FAST24, 2, kPrepWaves>(a, K == 2 * kWg, st);
        } else {
            launch_rows<BF16, NORM, M, FAST24, 4, kPrepWaves>(a, K == 4 * kWg, st);
        }
        if (a.global_scale) hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, a.global_scale, 1.0f);
        return hipGetLastError();
    }
    RowStats *stats = reinterpret_cast<RowStats *>(ws);
    if constexpr (FMT == kFmtNv) {
        // one row per workgroup while the row fits in registers (norm rows up
        // to 8192 elements, rows without norm up to 32768)
        const dim3 rows((unsigned)round_up8(a.T));
        constexpr int64_t kWg = (int64_t)kChunk * kPrepWaves;
        if (K <= kWg * 2)
            hipLaunchKernelGGL((k_nv_rowstats_wg<BF16, NORM, 2>), rows, blk, 0, st, a, stats);
        else if (K <= kWg * 4)
            hipLaunchKernelGGL((k_nv_rowstats_wg<BF16, NORM, 4>), rows, blk, 0, st, a, stats);
        else {
            bool done = false;
            if constexpr (NORM == kNormNone) {
                if (K <= kWg * 8) {
                    hipLaunchKernelGGL((k_nv_rowstats_wg<BF16, NORM, 8>), rows, blk, 0, st, a, stats);
                    done = true;
                } else if (K <= kWg * 16) {
                    hipLaunchKernelGGL((k_nv_rowstats_wg<BF16, NORM, 16>), rows, blk, 0, st, a, stats);
                    done = true;
                }
            }
            if (!done)
                hipLaunchKernelGGL((k_nv_rowstats<BF16, NORM>), dim3((unsigned)((a.T + kPrepWaves - 1) / kPrepWaves)),
                                   blk, 0, st, a, stats);
        }
        hipLaunchKernelGGL(k_nv_tensor_scale, dim3(1), dim3(1024), 0, st, stats, a.T, a.global_scale);
    } else if (a.global_scale) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, a.global_scale, 1.0f);
    }
    const int64_t tasks_per_row = (K + (int64_t)kChunk * kStreamChunks - 1) / ((int64_t)kChunk * kStreamChunks);
    const int64_t tasks = a.T * tasks_per_row;
    // one task per wave: measured fastest on MI355X for every shape tried
    // (more resident waves hide the load latency better than an in-wave
    // prefetch of a next task)
    const int64_t waves = tasks;
    const dim3 grid((unsigned)round_up8((waves + kPrepWaves - 1) / kPrepWaves));
    if constexpr (FMT == kFmtNv || NORM == kNormNone) {
        if (a.off32)
            hipLaunchKernelGGL((k_prep_stream<BF16, NORM, FMT, M, FAST24, true>), grid, blk, 0, st, a, stats);
        else
            hipLaunchKernelGGL((k_prep_stream<BF16, NORM, FMT, M, FAST24, false>), grid, blk, 0, st, a, stats);
    }
    return hipGetLastError();
}

template <bool BF16, int NORM, int FMT>
static hipError_t launch_prep_m(const PrepArgs &a, void *ws, hipStream_t st) {
    if (a.m == 4 && a.n == 2) return launch_prep_t<BF16, NORM, FMT, 4, 1>(a, ws, st);
    switch (a.m) {
        case 1: return launch_prep_t<BF16, NORM, FMT, 1, 0>(a, ws, st);
        case 2: return launch_prep_t<BF16, NORM, FMT, 2, 0>(a, ws, st);
        case 4: return launch_prep_t<BF16, NORM, FMT, 4, 0>(a, ws, st);
        case 8: return launch_prep_t<BF16, NORM, FMT, 8, 0>(a, ws, st);
        case 16: return launch_prep_t<BF16, NORM, FMT, 16, 0>(a, ws, st);
    }
    return hipErrorInvalidValue;
}

template <bool BF16, int NORM>
static hipError_t launch_prep_f(const PrepArgs &a, void *ws, hipStream_t st) {
    return a.fmt == kFmtMx ? launch_prep_m<BF16, NORM, kFmtMx>(a, ws, st)
                           : launch_prep_m<BF16, NORM, kFmtNv>(a, ws, st);
}

template <bool BF16>
static hipError_t launch_prep_n(const PrepArgs &a, void *ws, hipStream_t st) {
    switch (a.norm) {
        case kNormNone: return launch_prep_f<BF16, kNormNone>(a, ws, st);
        case kNormRms: return launch_prep_f<BF16, kNormRms>(a, ws, st);
        case kNormLayer: return launch_prep_f<BF16, kNormLayer>(a, ws, st);
    }
    return hipErrorInvalidValue;
}

template <int FMT, int M, int FAST24>
static hipError_t launch_swiglu_t(const PrepArgs &a, void *ws, hipStream_t st) {
    const dim3 blk(kPrepWaves * kWave);
    if constexpr (FMT == kFmtNv) {
        RowStats *stats = reinterpret_cast<RowStats *>(ws);
        hipLaunchKernelGGL(k_swiglu_rowstats, dim3((unsigned)((a.T + kPrepWaves - 1) / kPrepWaves)), blk, 0, st, a,
                           stats);
        hipLaunchKernelGGL(k_nv_tensor_scale, dim3(1), dim3(1024), 0, st, stats, a.T, a.global_scale);
    } else if (a.global_scale) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, a.global_scale, 1.0f);
    }
    const int64_t tpr = (a.K + (int64_t)kChunk * kSwiChunks - 1) / ((int64_t)kChunk * kSwiChunks);
    const int64_t tasks = a.T * tpr;
    const dim3 grid((unsigned)round_up8((tasks + kPrepWaves - 1) / kPrepWaves));
    hipLaunchKernelGGL((k_prep_swiglu<FMT, M, FAST24>), grid, blk, 0, st, a);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_swiglu_m(const PrepArgs &a, void *ws, hipStream_t st) {
    if (a.m == 4 && a.n == 2) return launch_swiglu_t<FMT, 4, 1>(a, ws, st);
    switch (a.m) {
        case 1: return launch_swiglu_t<FMT, 1, 0>(a, ws, st);
        case 2: return launch_swiglu_t<FMT, 2, 0>(a, ws, st);
        case 4: return launch_swiglu_t<FMT, 4, 0>(a, ws, st);
        case 8: return launch_swiglu_t<FMT, 8, 0>(a, ws, st);
        case 16: return launch_swiglu_t<FMT, 16, 0>(a, ws, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prepare_swiglu(const PrepArgs &a, void *ws, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    return a.fmt == kFmtMx ? launch_swiglu_m<kFmtMx>(a, ws, st) : launch_swiglu_m<kFmtNv>(a, ws, st);
}

hipError_t launch_prepare(const PrepArgs &a, void *ws, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    return a.bf16 ? launch_prep_n<true>(a, ws, st) : launch_prep_n<false>(a, ws, st);
}

size_t prepare_workspace_bytes(int64_t T, int fmt) {
    return fmt == kFmtNv ? (size_t)(T > 0 ? T : 1) * sizeof(RowStats) : 0;
}

// ---------------------------------------------------------------- allocation-free preparation
// Scratch of sharq_prepare_noalloc: the NVFP4 per-row statistics of up to
// kNoallocRows rows, in a file-scope device array that every GPU the library
// runs on holds until the process ends.  Host code never passes the array's
// name (a host-side stand-in, not a device address) to a kernel: the device
// address is looked up once per device, with that device current, and kept.
// Every call on a device shares its array, so calls that overlap on one GPU
// race; nothing in it has to start at zero (each launch writes every row's
// statistics before the tensor-scale kernel reads them).
static_assert(kNoallocRows * sizeof(RowStats) <= ((size_t)1 << 20), "scratch stays at 1 MiB");
static __device__ __align__(256) RowStats scratch[kNoallocRows];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {nullptr};

hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_prepare_noalloc(const PrepArgs &a, hipStream_t st) {
    if (a.T == 0) return hipSuccess;
    void *ws = nullptr;
    if (a.fmt == kFmtNv) {
        if (a.T > kNoallocRows) return hipErrorInvalidValue;  // the entry point rejects this first
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) return e;
    }
    return launch_prepare(a, ws, st);
}

}  // namespace sharq
