// Device helpers shared by the gfx950 kernels: bf16 packing, wavefront
// folds, and the fixed summation order of the square sum.
//
// Arithmetic rules for every kernel of this library (built with
// -ffp-contract=off, denormals on, IEEE division and square root):
//   * bf16 -> float32 widening is exact (a shift);
//   * each float32 operation rounds to nearest even once; no contraction;
//   * float32 -> bf16 rounds to nearest even once, at the store
//     (v_cvt_pk_bf16_f32 on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Streaming inputs (kv rows, cos/sin rows, read exactly once) are loaded with
// the non-temporal hint, which keeps them from displacing the shared gamma
// row and the indices in the caches. (Cache rows are written through L2 with
// sc1 stores where the caches fit a buffer descriptor: the non-temporal hint
// made those writes slower on MI355X.)
#ifndef KVRC_NT_LOADS
#define KVRC_NT_LOADS 1
#endif

namespace kvrc {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T stream_load(const void *p)
{
#if KVRC_NT_LOADS
    return __builtin_nontemporal_load(static_cast<const T *>(p));
#else
    return *static_cast<const T *>(p);
#endif
}

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ u32x4 to_u32x4(uint4 v) { return u32x4{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ uint2 to_uint2(u32x2 v) { return make_uint2(v.x, v.y); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two float32 values -> two bf16 (round to nearest even) packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Eight bf16 (one 16-byte chunk) -> float32.
__device__ __forceinline__ void unpack8(const uint4 &q, float (&x)[8])
{
    x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x);
    x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
    x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z);
    x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
}

__device__ __forceinline__ uint4 pack8(const float (&y)[8])
{
    uint4 q;
    q.x = pack_bf16x2(y[0], y[1]);
    q.y = pack_bf16x2(y[2], y[3]);
    q.z = pack_bf16x2(y[4], y[5]);
    q.w = pack_bf16x2(y[6], y[7]);
    return q;
}

// Square sum of one 8-element chunk in element order, starting from acc:
// each square is rounded, then added (no fused multiply-add).
__device__ __forceinline__ float chunk_sumsq(const float (&x)[8], float acc)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float sq = x[e] * x[e];
        acc = acc + sq;
    }
    return acc;
}

// Fold a value across groups of G lanes (G a power of two <= 64) by halves:
// step masks G/2, G/4, ..., 1. With partial p[l] in lane l of the group, the
// result (in every lane of the group) is the halving tree
//   p[k] <- p[k] + p[k + w/2], w = G, G/2, ..., 2
// because lane k and lane k ^ m hold the two operands and float addition is
// commutative.
//
// The exchanges stay on the vector ALU (no LDS round trip):
//   m = 32: v_permlane32_swap of the value with itself leaves the lower half
//           in one result and the upper half in the other, in every lane;
//   m = 16: v_permlane16_swap likewise pairs rows 0/1 and 2/3 of 16 lanes;
//   m = 8:  DPP row rotate by 8 (lane l reads lane l ^ 8 within its row);
//   m = 4:  DPP row rotate by 4 reads lane l + 4 or l - 4 (mod 16), which
//           after the m = 8 step holds the same value as lane l ^ 4;
//   m = 2, 1: DPP quad permutes [2,3,0,1] and [1,0,3,2].
// Below G = 16 the m = 4 step needs the exact partner and uses a shuffle.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_read(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, false);
}

template <int G, typename Op>
__device__ __forceinline__ uint32_t fold_lanes(uint32_t v, Op op)
{
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G: power of two <= 64");
    if constexpr (G == 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = op(r[0], r[1]);
    }
    if constexpr (G >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = op(r[0], r[1]);
    }
    if constexpr (G >= 16) {
        v = op(v, dpp_read<0x128>(v));            // row_ror:8
        v = op(v, dpp_read<0x124>(v));            // row_ror:4
    } else if constexpr (G >= 8) {
        v = op(v, (uint32_t)__shfl_xor((int)v, 4, 64));
    }
    if constexpr (G >= 4)
        v = op(v, dpp_read<0x4E>(v));             // quad_perm [2,3,0,1]
    if constexpr (G >= 2)
        v = op(v, dpp_read<0xB1>(v));             // quad_perm [1,0,3,2]
    return v;
}

struct FloatAdd {
    __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const
    {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }
};
struct UnsignedMax {
    __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const
    {
        return a > b ? a : b;
    }
};

template <int G>
__device__ __forceinline__ float fold_sum(float v)
{
    return __uint_as_float(fold_lanes<G>(__float_as_uint(v), FloatAdd{}));
}

// Maximum of values that are >= +0 and not NaN (an fmaxf chain started at 0
// never yields NaN): for those, float order is the unsigned order of the
// bits, which keeps the fold free of NaN canonicalisation.
template <int G>
__device__ __forceinline__ float fold_max(float v)
{
    return __uint_as_float(fold_lanes<G>(__float_as_uint(v), UnsignedMax{}));
}

// ---------------------------------------------------------------------------
// Correctly rounded division with a shared divisor.
//
// q = RN(a / b) for many a and one b > 0: with rb = RN(1/b) from one IEEE
// division, two Newton-Raphson corrections of the quotient
//   q0 = RN(a * rb)
//   q1 = RN(q0 + RN(a - q0*b) * rb)      (q1 is within one ulp of a/b)
//   q2 = RN(q1 + (a - q1*b) * rb)        (a - q1*b is exact in an fma)
// give q2 = RN(a / b) (Markstein's theorem: a faithful quotient corrected with
// the correctly rounded reciprocal and the exact remainder rounds correctly),
// provided no intermediate leaves the normal range. That holds on the domain
//   2^-60 <= b <= 2^60  and  2^-64 <= |a| <= 2^66:
// the quotient lies in [2^-124, 2^126], and the remainder a - q*b is zero or a
// multiple of ulp(q)*ulp(b) > 2^-48 |a| >= 2^-112, hence normal.
// Callers test the domain and use IEEE division outside it.
// Five VALU operations per quotient instead of eleven.
// ---------------------------------------------------------------------------
constexpr float kFastDivLo = 0x1p-60f;
constexpr float kFastDivHi = 0x1p60f;
constexpr float kFastDivDividendLo = 0x1p-64f;
// Bit pattern of 2^-120: a square x*x at or above it means |x| >= 2^-60.
constexpr uint32_t kMinSquareBits = 0x03800000u;

__device__ __forceinline__ bool fast_div_divisor_ok(float b)
{
    return b >= kFastDivLo && b <= kFastDivHi;    // false for NaN
}

// RN(1/b) for 2^-60 <= b <= 2^60 without the IEEE division sequence: the
// hardware estimate y0 (v_rcp_f32, within one ulp of 1/b) and one
// Newton-Raphson correction with the residual e = 1 - b*y0 (exact in an fma
// when y0 is that close), y1 = RN(y0 + y0*e). Three VALU operations instead
// of about eleven; the self-test kvrc_selftest_recip lets a test compare it
// with IEEE division for every float32 of the domain.
__device__ __forceinline__ float rcp_rn(float b)
{
    const float y0 = __builtin_amdgcn_rcpf(b);
    const float e = __builtin_fmaf(-b, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

__device__ __forceinline__ float div_rn_shared(float a, float b, float rb)
{
    float q = a * rb;
    float r = __builtin_fmaf(-q, b, a);
    q = __builtin_fmaf(r, rb, q);
    r = __builtin_fmaf(-q, b, a);
    return __builtin_fmaf(r, rb, q);
}

// RN(amax / d) for a row maximum amax >= 0 and a constant divisor d (127 or
// 448): the shared-divisor quotient with RN(1/d) folded by the compiler when
// amax lies in its dividend domain, IEEE division otherwise (0, tiny, huge).
__device__ __forceinline__ float row_scale(float amax, float d)
{
    if (amax >= kFastDivDividendLo && amax <= 0x1p66f)
        return div_rn_shared(amax, d, 1.0f / d);
    return amax / d;
}

// 1.5 * 2^23: for |q| < 2^22, RN(q + kRoundMagic) = kRoundMagic + rint(q)
// (ties to even), so the low byte of its bits is rint(q) as an int8.
constexpr float kRoundMagic = 12582912.0f;

// Low bytes of eight words -> eight consecutive bytes (v_perm_b32).
__device__ __forceinline__ u32x2 pack_low_bytes8(const uint32_t (&w)[8])
{
    // perm(hi, lo, sel): selector byte k picks byte k of lo (0-3) or of hi (4-7);
    // 0x0c yields a zero byte.
    const uint32_t a = __builtin_amdgcn_perm(w[1], w[0], 0x0c0c0400u);   // b0 b1 0 0
    const uint32_t b = __builtin_amdgcn_perm(w[3], w[2], 0x04000c0cu);   // 0 0 b2 b3
    const uint32_t c = __builtin_amdgcn_perm(w[5], w[4], 0x0c0c0400u);
    const uint32_t d = __builtin_amdgcn_perm(w[7], w[6], 0x04000c0cu);
    return u32x2{a | b, c | d};
}

// Four float32 values -> four FLOAT8 E4M3FN codes (OCP format: 4 exponent
// bits with bias 7, 3 mantissa bits, largest finite value 448, no
// infinities), bytes 0..3 of the result in argument order: each value is
// rounded to the nearest E4M3FN value, ties to the even code, with the sign
// of the input (v_cvt_pk_fp8_f32, which on gfx950 converts to the OCP format
// with round to nearest even). Valid for |x| < 464: up to there the nearest
// value under that rounding is at most 448, the largest code (464 is the
// midpoint between 448 and 480, where the format has no finite value).
// Callers clamp (e4m3_clamp) wherever a value can reach 464.
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float e4m3_clamp(float x)
{
    return __builtin_amdgcn_fmed3f(x, -kE4m3Max, kE4m3Max);    // keeps the sign of zero
}

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Distance key of t (a normal float32 with |t| >= 2^-6) from the midpoints
// between neighbouring E4M3FN values: below kE4m3NearKey exactly when t lies
// within [-4, +3] float32 ulps of a midpoint. In that range every E4M3FN
// value has 3 mantissa bits, so the midpoints are the floats whose 20 low
// mantissa bits are 0x80000; the midpoints sit mid-binade, so t, the midpoint
// and anything a few ulps from them share one binade. The key is the low 20
// bits of bits(t) + 4 - 0x80000 moved to the top, so a minimum over many t
// answers for all of them at once.
__device__ __forceinline__ uint32_t e4m3_midpoint_key(float t)
{
    return (__float_as_uint(t) + (4u - 0x80000u)) << 12;
}
constexpr uint32_t kE4m3NearKey = 8u << 12;

__device__ __forceinline__ u32x2 e4m3_pack8(const float (&q)[8])
{
    return u32x2{e4m3_pack4(q[0], q[1], q[2], q[3]), e4m3_pack4(q[4], q[5], q[6], q[7])};
}

// Pack eight int8 codes (given as float integral values in [-127, 127]).
__device__ __forceinline__ uint2 pack_codes8(const float (&c)[8])
{
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = (uint32_t)((int32_t)c[e]) & 0xffu;
    uint2 r;
    r.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    r.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return r;
}

}  // namespace kvrc
