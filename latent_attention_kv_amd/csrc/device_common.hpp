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

namespace kvrc {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
template <int G>
__device__ __forceinline__ float fold_sum(float v)
{
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1)
        v = v + __shfl_xor(v, m, 64);
    return v;
}

template <int G>
__device__ __forceinline__ float fold_max(float v)
{
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
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
