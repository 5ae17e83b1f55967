// Device helpers shared by the gfx950 kernels of the SharQ hot path.
//
// Element formats (OCP MX v1.0 for E2M1/E8M0; E4M3 as used by NVFP4):
//   E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, code bit 3 = sign;
//   E8M0 byte b = 2^(b-127); E4M3 bias 7, 3 fraction bits, max 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- 16-bit loads
// Two 16-bit elements packed in a 32-bit word, element 0 in the low half.
template <bool BF16>
__device__ __forceinline__ float elem_lo(uint32_t w) {
    if constexpr (BF16) {
        return __uint_as_float(w << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    }
}
template <bool BF16>
__device__ __forceinline__ float elem_hi(uint32_t w) {
    if constexpr (BF16) {
        return __uint_as_float(w & 0xFFFF0000u);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
}

// Eight consecutive elements from one 128-bit word.
template <bool BF16>
__device__ __forceinline__ void unpack8(const uint4 &q, float v[8]) {
    v[0] = elem_lo<BF16>(q.x); v[1] = elem_hi<BF16>(q.x);
    v[2] = elem_lo<BF16>(q.y); v[3] = elem_hi<BF16>(q.y);
    v[4] = elem_lo<BF16>(q.z); v[5] = elem_hi<BF16>(q.z);
    v[6] = elem_lo<BF16>(q.w); v[7] = elem_hi<BF16>(q.w);
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources: loads at offsets >= the resource's byte count return
// zeros, so out-of-range rows of a tile need no branch.  Offsets are 32-bit;
// the C ABI keeps every operand below 2 GiB.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Direct buffer -> LDS loads: lane i's bytes land at lds + i*size (lds is
// wave-uniform); out-of-range lanes write zeros.  The byte offset is the
// per-lane voff plus the wave-uniform soff; callers keep voff + soff below
// 2^32 (an out-of-range lane has voff = 2^31 and soff < 2^31).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, uint32_t soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, soff, 0, 0);
}

// ---------------------------------------------------------------- XCD-aware grids
// Workgroups are dealt to the eight XCDs round-robin (id % 8).  Block b of a
// grid of nb blocks (nb a multiple of 8) -> logical block index such that
// every XCD runs one contiguous range of logical blocks.  Neighbouring rows,
// which share cache lines of the K-tiled outputs, then go through one L2.
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb) { return (b % 8) * (nb / 8) + b / 8; }

__host__ __device__ inline int64_t round_up8(int64_t n) { return (n + 7) / 8 * 8; }

// ---------------------------------------------------------------- lane exchange
// DPP quad permutations: lane i of every group of four reads lane perm[i].
constexpr int kDppQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// Same permutation with bound_ctrl set (every quad source lane exists, so the
// result is identical); this form folds into the consuming VALU instruction.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32_bc(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

constexpr int kDppRowMirror = 0x140;      // lane i of a row of 16 reads lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i of a half row of 8 reads lane 7 - i

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Sum of v over the 64 lanes of a fully active wave, the same value in every
// lane, always in the same order: pairs, quads, half rows and rows by DPP
// (both lanes of each exchange add the same two values, so every lane of a
// row holds the identical row sum), then (row0 + row1) + (row2 + row3).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<kDppQuadXor1>(v);
    v += dpp_f64<kDppQuadXor2>(v);
    v += dpp_f64<kDppRowHalfMirror>(v);
    v += dpp_f64<kDppRowMirror>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ---------------------------------------------------------------- E2M1
// Round |u| to the E2M1 grid (nearest, ties to even, saturating at 6).
// Returns the 3-bit magnitude code and the rounded magnitude.
// For |u| >= 1 the float is rounded to one fraction bit in its own binade by
// integer arithmetic on the bit pattern; below 1 the grid step is 0.5.
__device__ __forceinline__ uint32_t e2m1_round(float u, float &qmag) {
    const uint32_t b = __float_as_uint(u) & 0x7FFFFFFFu;
    const float a = __uint_as_float(b);
    uint32_t code;
    if (a >= 1.0f) {
        const uint32_t r = (b + 0x1FFFFFu + ((b >> 22) & 1u)) >> 22;  // exponent:1-bit fraction
        code = min(r - 252u, 7u);                                        // 1.0 -> 254 -> code 2
        qmag = code == 7u ? 6.0f : __uint_as_float(r << 22);
    } else {
        code = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f);
        qmag = 0.5f * (float)code;
    }
    return code;
}

// Signed 4-bit code of u (canonical +0 for a zero magnitude) and the signed
// rounded value (+0 when the code is 0).
__device__ __forceinline__ uint32_t e2m1_encode(float u, float &q) {
    float qmag;
    uint32_t c = e2m1_round(u, qmag);
    const uint32_t neg = (c != 0u) ? (__float_as_uint(u) >> 31) : 0u;
    q = __uint_as_float(__float_as_uint(qmag) | (neg << 31));
    return c | (neg << 3);
}

// Hardware E2M1 conversion of eight values (element i -> nibble i) divided
// by a power-of-two scale.  The scale operand carries an E8M0 exponent E as
// the float bit pattern (E+127) << 23 (so 2^-127 is the pattern 0).
// v_cvt_scalef32_pk_fp4_f32 then yields the nearest-even, saturating E2M1
// code of v*2^-E, except that a negative value rounding to zero keeps its
// sign (code 0x8); those sign bits are cleared so that a zero magnitude is
// always the code 0x0.  At unit scale the result equals nearest-even
// rounding on every one of the 2^32 float32 inputs (measured on MI355X).
__device__ __forceinline__ uint32_t e2m1_cvt8(const float u[8], float scale) {
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, u[0], u[1], scale, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, u[2], u[3], scale, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, u[4], u[5], scale, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, u[6], u[7], scale, 3);
    // adding 7 to each nibble's 3-bit magnitude carries into its sign
    // position exactly when the magnitude is non-zero
    const uint32_t nz = (p & 0x77777777u) + 0x77777777u;
    return p & (nz | 0x77777777u);
}

typedef float sharq_v2f __attribute__((ext_vector_type(2)));

// Values of eight E2M1 codes times the power-of-two scale (same encoding as
// above); exact, +0 for code 0.
__device__ __forceinline__ void e2m1_dec8(uint32_t p, float scale, float q[8]) {
    sharq_v2f t;
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, scale, 0); q[0] = t.x; q[1] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, scale, 1); q[2] = t.x; q[3] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, scale, 2); q[4] = t.x; q[5] = t.y;
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, scale, 3); q[6] = t.x; q[7] = t.y;
}

// E8M0 exponent E as the scale operand of the conversions above.
__device__ __forceinline__ float e8m0_operand(int E) { return __uint_as_float((uint32_t)(E + 127) << 23); }

// Double reciprocal of a positive finite double d whose inverse is a normal
// double (every positive float qualifies): the hardware reciprocal refined
// by two Newton steps r <- r + r(1 - dr), each an FMA pair.  From a start
// within 2^-20 the first step leaves about 2^-40 and the second the final
// rounding (2^-53) plus 2^-79, so the result is within one ulp of the
// correctly rounded 1/d.  No range scaling is needed for such d.
__device__ __forceinline__ double rcp_f64_refined(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = __fma_rn(r, __fma_rn(-d, r, 1.0), r);
    return __fma_rn(r, __fma_rn(-d, r, 1.0), r);
}

// ---------------------------------------------------------------- E8M0 (MX)
// OCP MX shared exponent for E2M1 elements: floor(log2 amax) - 2, or -127
// for amax == 0 (never below -127; at most 125 for finite floats).  The
// frexp exponent of a finite a > 0 (subnormals included) is floor(log2 a)+1.
__device__ __forceinline__ int mx_shared_exp(float amax) {
    const int e = __builtin_amdgcn_frexp_expf(amax) - 3;
    return amax == 0.0f ? -127 : (e < -127 ? -127 : e);
}

// Max over the four lanes of a quad (MX block) / a lane pair (NVFP4 block)
// of a non-negative float, done on the bit pattern (same order as the value).
__device__ __forceinline__ float quad_max_nonneg(float m) {
    uint32_t b = __float_as_uint(m);
    b = max(b, dpp_u32_bc<kDppQuadXor1>(b));
    b = max(b, dpp_u32_bc<kDppQuadXor2>(b));
    return __uint_as_float(b);
}
__device__ __forceinline__ float pair_max_nonneg(float m) {
    uint32_t b = __float_as_uint(m);
    b = max(b, dpp_u32_bc<kDppQuadXor1>(b));
    return __uint_as_float(b);
}

// 2^-E as a normal float for E in [-127, 125].
__device__ __forceinline__ float pow2_neg(int E) { return __uint_as_float((uint32_t)(127 - E) << 23); }

// ---------------------------------------------------------------- E4M3 (NVFP4 scales)
// Nearest E4M3 (ties to even), saturating at 448; t >= 0 and finite.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float t) {
    if (!(t > 0.0f)) return 0u;
    if (t >= 448.0f) return 0x7Eu;
    const uint32_t b = __float_as_uint(t);
    if (b < 0x3C800000u) {                      // t < 2^-6: subnormal step 2^-9
        return (uint32_t)__builtin_rintf(t * 512.0f);  // 8 lands on 0x08 = 2^-6
    }
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;  // 3 fraction bits, RNE
    return ((r >> 3) - 120u) << 3 | (r & 7u);
}

__device__ __forceinline__ float e4m3_value(uint32_t s) {
    const uint32_t e = (s >> 3) & 15u, f = s & 7u;
    return e == 0u ? (float)f * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (f << 20));
}

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

// ---------------------------------------------------------------- SiLU(gate) * up source
// The activation of a down projection computed from the gate/up product's
// float rows: x = fl32(SiLU(gate) * up), SiLU(g) = g / (1 + e^-g), with e^y
// evaluated by fixed correctly rounded float steps: Cody-Waite reduction
// y = n ln2 + r (n = rint(y log2 e), ln2 as a 15-bit head plus a tail), the
// degree-6 Taylor polynomial of e^r in Horner form (one fused multiply-add
// per step), scaling by 2^n; 0 below
// -87 (never subnormal), +inf above 88.
__device__ __forceinline__ float exp32_fixed(float y) {
    if (!(y <= 88.0f)) return __builtin_inff();
    if (y < -87.0f) return 0.0f;
    const float n = __builtin_rintf(__fmul_rn(y, 1.44269504f));
    const float r = __fsub_rn(__fsub_rn(y, __fmul_rn(n, 0.693145752f)), __fmul_rn(n, 1.42860677e-6f));
    float p = 0.00138888889f;                 // 1/720
    p = __builtin_fmaf(p, r, 0.00833333333f);  // 1/120
    p = __builtin_fmaf(p, r, 0.0416666667f);   // 1/24
    p = __builtin_fmaf(p, r, 0.166666667f);    // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float silu_times(float g, float u) {
    const float d = __fadd_rn(1.0f, exp32_fixed(-g));
    return __fmul_rn(__fdiv_rn(g, d), u);
}

// The same value for |g| <= 80, in fewer instructions.  e^-g: no range
// tests (-g lies inside [-87, 88]), and y - n * ln2_head as one fused
// multiply-add, the same number because n * ln2_head is exact (|n| <= 116
// and a 15-bit head).  g / d (1 <= d <= 1 + e^80, far from overflow and
// underflow): the product of g and the hardware reciprocal (within 1 ulp of
// 1/d), corrected once by its exact remainder g - q0 * d, sign taken from g.
// That is not a correctly rounded division for arbitrary operands, but for
// the divisors 1 + e^-g it is: the result equals the oracle's correctly
// rounded quotient on every float32 g of the range (checked exhaustively on
// the GPU).
__device__ __forceinline__ float silu_times_inrange(float g, float u) {
    const float y = -g;
    const float n = __builtin_rintf(__fmul_rn(y, 1.44269504f));
    const float r = __fsub_rn(__builtin_fmaf(-n, 0.693145752f, y), __fmul_rn(n, 1.42860677e-6f));
    float p = 0.00138888889f;
    p = __builtin_fmaf(p, r, 0.00833333333f);
    p = __builtin_fmaf(p, r, 0.0416666667f);
    p = __builtin_fmaf(p, r, 0.166666667f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float d = __fadd_rn(1.0f, __builtin_ldexpf(p, (int)n));
    const float z = __builtin_amdgcn_rcpf(d);
    const float q0 = __fmul_rn(g, z);
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, d, g), z, q0);
    return __fmul_rn(__builtin_copysignf(q, g), u);  // g = -0: the correction's sum gives +0
}

// h[k] = silu_times(g[k], u[k]) for N values per lane: the short form when
// every value of every active lane lies in [-80, 80] (a wave-uniform
// branch), else the general one.
template <int N>
__device__ __forceinline__ void silu_times_n(const float *g, const float *u, float *h) {
    bool in = true;
#pragma unroll
    for (int k = 0; k < N; k++) in = in && fabsf(g[k]) <= 80.0f;  // false for NaN
    if (__all(in)) {
#pragma unroll
        for (int k = 0; k < N; k++) h[k] = silu_times_inrange(g[k], u[k]);
    } else {
#pragma unroll
        for (int k = 0; k < N; k++) h[k] = silu_times(g[k], u[k]);
    }
}

}  // namespace sharq
