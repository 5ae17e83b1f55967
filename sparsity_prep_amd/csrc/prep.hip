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
//   MX + norm, K <= 8192:  a workgroup of four waves per row (from 2048 rows
//                          on, 2 or 4 consecutive rows per workgroup, the
//                          next row loaded during the current one); the row
//                          stays in registers across the FP64 norm reduction
//                          (whose per-wave partials meet in LDS) and the
//                          quantization pass;
//   MX + norm, larger K:   one wave per row, the quantization pass re-reads
//                          the row (L2 hit);
//   no norm:               tasks are (row, group of chunks), fully parallel;
//   NVFP4:                 a pre-pass writes per-row norm statistics and
//                          amax, a one-block kernel reduces the tensor scale,
//                          then the main pass streams (row, chunk-group) tasks.
#include "device_util.h"
#include "kernels.h"

namespace sharq {

constexpr int kPrepWaves = 4;        // waves per workgroup
constexpr int kChunk = 512;          // elements per wave-wide 128-bit load
constexpr int kStreamChunks = 2;     // chunks per task when rows are split (measured: 2 beats 4 and 8)
constexpr int64_t kPrepRowsGrid = 1024;   // row workgroups that fill the GPU (four per CU)

struct RowStats {  // per-row statistics written by the NVFP4 pre-pass
    float r, mu, amax, pad;
};

// ---------------------------------------------------------------- selection
// keep bit i of the result is set when element i (of the 8 owned by the lane)
// is among the N largest magnitudes of its M-group; equal magnitudes favour
// the lower index.  M in {1,2,4,8}: groups lie inside the lane.
template <int M>
__device__ __forceinline__ uint32_t select_in_lane(const float v[8], int n) {
    uint32_t key[8];
#pragma unroll
    for (int i = 0; i < 8; i++) key[i] = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    uint32_t keep = 0;
#pragma unroll
    for (int g = 0; g < 8; g += M) {
#pragma unroll
        for (int i = 0; i < M; i++) {
            int rank = 0;
#pragma unroll
            for (int j = 0; j < M; j++) {
                if (j == i) continue;
                const bool beats = j < i ? key[g + j] >= key[g + i] : key[g + j] > key[g + i];
                rank += beats ? 1 : 0;
            }
            keep |= (rank < n ? 1u : 0u) << (g + i);
        }
    }
    return keep;
}

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

// 2:4 (the workloads' pattern): element i is kept iff it beats at least two
// of the three others.  The six magnitude comparisons (|a| >= |b| on floats,
// which orders finite values, subnormals and +-0 exactly like the bit
// patterns without sign) are taken as wave-wide lane masks (ballot), the
// majority logic runs on those masks in scalar registers, and each lane reads
// its keep flags back as lane masks (inverse ballot) to select the kept
// values, so no per-lane 0/1 values are materialized.  Inactive lanes
// contribute 0 bits and never read theirs.
__device__ __forceinline__ void select_2of4(const float v[8], uint64_t km[8]) {
#pragma unroll
    for (int g = 0; g < 8; g += 4) {
        const float a0 = fabsf(v[g]), a1 = fabsf(v[g + 1]), a2 = fabsf(v[g + 2]), a3 = fabsf(v[g + 3]);
        // lower index wins ties
        const uint64_t c01 = __builtin_amdgcn_ballot_w64(a0 >= a1), c02 = __builtin_amdgcn_ballot_w64(a0 >= a2);
        const uint64_t c03 = __builtin_amdgcn_ballot_w64(a0 >= a3), c12 = __builtin_amdgcn_ballot_w64(a1 >= a2);
        const uint64_t c13 = __builtin_amdgcn_ballot_w64(a1 >= a3), c23 = __builtin_amdgcn_ballot_w64(a2 >= a3);
        km[g] = (c01 & c02) | (c01 & c03) | (c02 & c03);
        km[g + 1] = (~c01 & c12) | (~c01 & c13) | (c12 & c13);
        km[g + 2] = (~c02 & ~c12) | (~c02 & c23) | (~c12 & c23);
        km[g + 3] = (~c03 & ~c13) | (~c03 & ~c23) | (~c13 & ~c23);
    }
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
// the quotient, so both round to the same float.  A zero divisor gives the
// same infinities and NaNs as the division.
__device__ __forceinline__ uint32_t quant_nv8(const float s[8], float G, double rG6, uint32_t &codes,
                                              float deq[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(s[i]));
    m = pair_max_nonneg(m);
    const uint32_t sb = e4m3_encode_sat((float)((double)m * rG6));
    const float D = __fmul_rn(e4m3_value(sb), G);
    const double rD = 1.0 / (double)D;
    float u[8], q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) u[i] = sb != 0u ? (float)((double)s[i] * rD) : 0.0f;
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
// Per-lane constant parts of the K-tiled offsets of a wave-wide chunk (512
// elements, chunk index ch along K, which starts on a K-tile boundary): lane
// l writes K tile 4ch + l/16, elements (l%16)*8 .. +7 of it.  With these the
// byte offset of the lane's codes (scales) in the 32-bit path is
// ch * T * 256 (ch * T * 512/B) + row * 64 (row * 128/B) + co (so), a
// scalar base plus this constant.
struct LaneOff {
    uint32_t co, so;
};

template <int FMT>
__device__ __forceinline__ LaneOff lane_offsets(const PrepArgs &a, int lane) {
    constexpr uint32_t B = FMT == kFmtMx ? 32 : 16;
    const uint32_t q = (uint32_t)lane >> 4, w = ((uint32_t)lane & 15u) * 8u;
    return {q * (uint32_t)(a.T * (kTileK / 2)) + w / 2, q * (uint32_t)(a.T * (kTileK / B)) + w / B};
}

// Decompose eight consecutive normalized values (elements 8*lane .. +7 of
// chunk ch of `row`; row and ch wave-uniform) and store their share of the
// mask, codes and scales.
template <int FMT, int M, int FAST24>
__device__ __forceinline__ void decompose_store(const PrepArgs &a, int64_t row, int64_t ch, int lane, LaneOff lo,
                                                const float v[8], float G, double rG6) {
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
    if (a.mask) (a.mask + row * (K / 8) + ch * (kChunk / 8))[lane] = (uint8_t)keep;
    if (a.off32) {  // K % 128 == 0 and each array < 4 GiB
        const uint32_t cb = (uint32_t)ch * (uint32_t)(a.T * (kChunk / 2));
        const uint32_t sb = (uint32_t)ch * (uint32_t)(a.T * (kChunk / B));
        *reinterpret_cast<uint32_t *>(a.b_codes + row * (kTileK / 2) + cb + lo.co) = bc;
        *reinterpret_cast<uint32_t *>(a.r_codes + row * (kTileK / 2) + cb + lo.co) = rc;
        if ((lane % LPB) == 0) {
            (a.b_scales + row * (kTileK / B) + sb)[lo.so] = (uint8_t)bs;
            (a.r_scales + row * (kTileK / B) + sb)[lo.so] = (uint8_t)rs;
        }
    } else {
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

// ---------------------------------------------------------------- MX, norm, row split over a workgroup
// A workgroup of NWG waves handles `rpw` consecutive rows, one at a time;
// wave w owns chunks w, w+NWG, ... of a row (at most CPW of them, held in
// registers).  The next row's words are loaded before the current row is
// reduced and quantized, so its latency hides behind the current row's
// arithmetic.  Each wave reduces its FP64 partial sums, the NWG partials
// meet in LDS (two slots, alternating by row) and every wave adds them in
// the same fixed order, so all waves derive the same r (and mu).  gamma and
// beta are loaded once per workgroup.
template <bool BF16, int NORM, int M, int FAST24, int CPW, int NWG>
__global__ __launch_bounds__(NWG * kWave) void k_prep_mx_split(PrepArgs a, int64_t rpw) {
    __shared__ double part[2][2][NWG];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const LaneOff lo = lane_offsets<kFmtMx>(a, lane);
    const int64_t row0 = xcd_block(blockIdx.x, gridDim.x) * rpw;
    const int64_t row_end = row0 + rpw < a.T ? row0 + rpw : a.T;
    if (row0 >= row_end) return;
    const int64_t K = a.K;

    bool in[CPW];
    uint4 graw[CPW], braw[CPW], raw[CPW];
    constexpr uint32_t kOnePair = BF16 ? 0x3F803F80u : 0x3C003C00u;  // 1.0, 1.0
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int64_t e0 = ((int64_t)(wave + NWG * j) * kWave + lane) * 8;
        in[j] = e0 < K;
        raw[j] = in[j] ? *reinterpret_cast<const uint4 *>(a.x + row0 * a.ldx + e0) : make_uint4(0, 0, 0, 0);
        graw[j] = in[j] ? param_raw<true>(a.gamma, e0, kOnePair) : make_uint4(0, 0, 0, 0);
        braw[j] = in[j] ? param_raw<NORM == kNormLayer>(a.beta, e0, 0u) : make_uint4(0, 0, 0, 0);
    }
    for (int64_t row = row0; row < row_end; row++) {
        const int slot = (int)(row & 1);
        uint4 nraw[CPW];
        const bool more = row + 1 < row_end;
#pragma unroll
        for (int j = 0; j < CPW; j++) {
            const int64_t e0 = ((int64_t)(wave + NWG * j) * kWave + lane) * 8;
            nraw[j] = (more && in[j]) ? *reinterpret_cast<const uint4 *>(a.x + (row + 1) * a.ldx + e0)
                                      : make_uint4(0, 0, 0, 0);
        }
        float v[8];
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
                    unpack8<BF16>(raw[j], v);
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const double d = (double)v[i] - mud;
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
                float g[8], b[8];
                unpack8<BF16>(graw[j], g);
                unpack8<BF16>(braw[j], b);
                unpack8<BF16>(raw[j], v);
                normalize8<NORM>(v, g, b, r, mu);
                decompose_store<kFmtMx, M, FAST24>(a, row, wave + NWG * j, lane, lo, v, 1.0f, 6.0f);
            }
        }
#pragma unroll
        for (int j = 0; j < CPW; j++) raw[j] = nraw[j];
    }
}

// ---------------------------------------------------------------- MX, norm, one row per workgroup
// A workgroup of NWG waves handles one row; wave w owns chunks w, w+NWG, ...
// of it (at most CPW of them, held in registers from one batch of loads).
// Each wave reduces its FP64 partial sums, the NWG partials meet in LDS and
// every wave adds them in the same fixed order, so all waves derive the same
// r (and mu).  Used below kPrepRowsGrid * 2 rows, where it beats the split
// kernel run with one row per workgroup (measured on MI355X: about 15% at
// a few hundred rows).
template <bool BF16, int NORM, int M, int FAST24, int CPW, int NWG>
__global__ __launch_bounds__(NWG * kWave) void k_prep_mx_row(PrepArgs a) {
    __shared__ double part[2][NWG];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const LaneOff lo = lane_offsets<kFmtMx>(a, lane);
    const int64_t row = xcd_block(blockIdx.x, gridDim.x);
    if (row >= a.T) return;
    const int64_t K = a.K;

    bool in[CPW];
    uint4 graw[CPW], braw[CPW], raw[CPW];
    constexpr uint32_t kOnePair = BF16 ? 0x3F803F80u : 0x3C003C00u;  // 1.0, 1.0
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int64_t e0 = ((int64_t)(wave + NWG * j) * kWave + lane) * 8;
        in[j] = e0 < K;
        raw[j] = in[j] ? *reinterpret_cast<const uint4 *>(a.x + row * a.ldx + e0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int64_t e0 = ((int64_t)(wave + NWG * j) * kWave + lane) * 8;
        graw[j] = in[j] ? param_raw<true>(a.gamma, e0, kOnePair) : make_uint4(0, 0, 0, 0);
        braw[j] = in[j] ? param_raw<NORM == kNormLayer>(a.beta, e0, 0u) : make_uint4(0, 0, 0, 0);
    }
    float v[8];
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
    for (int w = 1; w < NWG; w++) s1 += part[0][w];
    float r, mu = 0.0f;
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
        for (int w = 1; w < NWG; w++) s2 += part[1][w];
        mu = (float)mud;
        r = (float)(1.0 / sqrt(s2 / (double)K + (double)a.eps));
    }
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        if (in[j]) {
            float g[8], b[8];
            unpack8<BF16>(graw[j], g);
            unpack8<BF16>(braw[j], b);
            unpack8<BF16>(raw[j], v);
            normalize8<NORM>(v, g, b, r, mu);
            decompose_store<kFmtMx, M, FAST24>(a, row, wave + NWG * j, lane, lo, v, 1.0f, 0.0);
        }
    }
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
            decompose_store<kFmtMx, M, FAST24>(a, row, ch, lane, lo, v, 1.0f, 0.0);
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

template <bool BF16, int NORM, int FMT, int M, int FAST24>
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
            decompose_store<FMT, M, FAST24>(a, row, c0 + c, lane, lo, v, G, rG6);
        }
    }
}

// ---------------------------------------------------------------- SiLU(gate) * up source
// The activation of a down projection computed from the gate/up product's
// float rows: x = fl32(SiLU(gate) * up), SiLU(g) = g / (1 + e^-g), with e^y
// evaluated by fixed correctly rounded float steps: Cody-Waite reduction
// y = n ln2 + r (n = rint(y log2 e), ln2 as a 15-bit head plus a tail), the
// degree-6 Taylor polynomial of e^r in Horner form, scaling by 2^n; 0 below
// -87 (never subnormal), +inf above 88.
__device__ __forceinline__ float exp32_fixed(float y) {
    if (!(y <= 88.0f)) return __builtin_inff();
    if (y < -87.0f) return 0.0f;
    const float n = __builtin_rintf(__fmul_rn(y, 1.44269504f));
    const float r = __fsub_rn(__fsub_rn(y, __fmul_rn(n, 0.693145752f)), __fmul_rn(n, 1.42860677e-6f));
    float p = 0.00138888889f;                      // 1/720
    p = __fadd_rn(__fmul_rn(p, r), 0.00833333333f);  // 1/120
    p = __fadd_rn(__fmul_rn(p, r), 0.0416666667f);   // 1/24
    p = __fadd_rn(__fmul_rn(p, r), 0.166666667f);    // 1/6
    p = __fadd_rn(__fmul_rn(p, r), 0.5f);
    p = __fadd_rn(__fmul_rn(p, r), 1.0f);
    p = __fadd_rn(__fmul_rn(p, r), 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float silu_times(float g, float u) {
    const float d = __fadd_rn(1.0f, exp32_fixed(-g));
    return __fmul_rn(__fdiv_rn(g, d), u);
}

// Eight activations at element e0 of a row from its gate and up words.
__device__ __forceinline__ void swiglu8(const float *row, int64_t K, int64_t e0, float v[8]) {
    const float4 g0 = *reinterpret_cast<const float4 *>(row + e0);
    const float4 g1 = *reinterpret_cast<const float4 *>(row + e0 + 4);
    const float4 u0 = *reinterpret_cast<const float4 *>(row + K + e0);
    const float4 u1 = *reinterpret_cast<const float4 *>(row + K + e0 + 4);
    v[0] = silu_times(g0.x, u0.x); v[1] = silu_times(g0.y, u0.y);
    v[2] = silu_times(g0.z, u0.z); v[3] = silu_times(g0.w, u0.w);
    v[4] = silu_times(g1.x, u1.x); v[5] = silu_times(g1.y, u1.y);
    v[6] = silu_times(g1.z, u1.z); v[7] = silu_times(g1.w, u1.w);
}

// (row, kStreamChunks chunks) tasks, one per wave.
template <int FMT, int M, int FAST24>
__global__ __launch_bounds__(kPrepWaves * kWave) void k_prep_swiglu(PrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = a.K;
    const int64_t tpr = (K + (int64_t)kChunk * kStreamChunks - 1) / ((int64_t)kChunk * kStreamChunks);
    const int64_t task = xcd_block(blockIdx.x, gridDim.x) * kPrepWaves + wave;
    const int64_t row = task / tpr;
    if (row >= a.T) return;
    const int64_t c0 = (task - row * tpr) * kStreamChunks;
    const float *gr = a.gu + row * a.ldgu;
    const LaneOff lo = lane_offsets<FMT>(a, lane);
    float G = 1.0f;
    double rG6 = 0.0;  // 1 / fl32(6G), NVFP4 only
    if constexpr (FMT == kFmtNv) {
        G = *a.global_scale;
        rG6 = 1.0 / (double)__fmul_rn(6.0f, G);
    }
#pragma unroll
    for (int c = 0; c < kStreamChunks; c++) {
        const int64_t e0 = (c0 + c) * kChunk + lane * 8;
        if (e0 < K) {
            float v[8];
            swiglu8(gr, K, e0, v);
            decompose_store<FMT, M, FAST24>(a, row, c0 + c, lane, lo, v, G, rG6);
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
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < T; i += blockDim.x) m = fmaxf(m, stats[i].amax);
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
template <bool BF16, int NORM, int FMT, int M, int FAST24>
static hipError_t launch_prep_t(const PrepArgs &a, void *ws, hipStream_t st) {
    const dim3 blk(kPrepWaves * kWave);
    const int64_t K = a.K;
    if constexpr (FMT == kFmtMx && NORM != kNormNone) {
        const dim3 grid((unsigned)round_up8((a.T + kPrepWaves - 1) / kPrepWaves));
        // rows per workgroup: about two workgroups per CU once T allows it;
        // below that one row per workgroup with all of its words loaded at once
        const int64_t rpw = a.T >= 4 * kPrepRowsGrid ? 4 : (a.T >= 2 * kPrepRowsGrid ? 2 : 1);
        const dim3 rows((unsigned)round_up8((a.T + rpw - 1) / rpw));
        // four waves of two chunks beat eight waves of one at K = 4096 (MI355X)
        if (K <= (int64_t)kChunk * kPrepWaves * 2) {
            if (rpw > 1)
                hipLaunchKernelGGL((k_prep_mx_split<BF16, NORM, M, FAST24, 2, kPrepWaves>), rows, blk, 0, st, a, rpw);
            else
                hipLaunchKernelGGL((k_prep_mx_row<BF16, NORM, M, FAST24, 2, kPrepWaves>), rows, blk, 0, st, a);
        } else if (K <= (int64_t)kChunk * kPrepWaves * 4) {
            if (rpw > 1)
                hipLaunchKernelGGL((k_prep_mx_split<BF16, NORM, M, FAST24, 4, kPrepWaves>), rows, blk, 0, st, a, rpw);
            else
                hipLaunchKernelGGL((k_prep_mx_row<BF16, NORM, M, FAST24, 4, kPrepWaves>), rows, blk, 0, st, a);
        }
        else
            hipLaunchKernelGGL((k_prep_mx_2pass<BF16, NORM, M, FAST24>), grid, blk, 0, st, a);
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
    if constexpr (FMT == kFmtNv || NORM == kNormNone)
        hipLaunchKernelGGL((k_prep_stream<BF16, NORM, FMT, M, FAST24>), grid, blk, 0, st, a, stats);
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
    const int64_t tpr = (a.K + (int64_t)kChunk * kStreamChunks - 1) / ((int64_t)kChunk * kStreamChunks);
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

}  // namespace sharq
