// Fused RMSNorm + interleaved RoPE + cache scatter for gfx950 (MI355X).
//
// Computes, per token (aclnnKvRmsNormRopeCache, Description and Formulas (1)
// interleaveRope, (2) rmsNorm; int8 rows use the RowMax(abs)/127 + round rule
// of aclnnMlaPrologV3WeightNz, Dequant Scale Query Nope formula, and FLOAT8
// E4M3FN rows, a ckv cache type of quantisation scenario 1, the same rule
// with 448, the largest E4M3FN value, in place of 127):
//   y  = (x / sqrt(sum(x*x)/Dv + eps)) * gamma          on kv[t, 0:Dv]
//   kr = cat(x1, x2) * cos + cat(-x2, x1) * sin          on kv[t, Dv:Dv+Dk]
//   ckv_cache[row] = bf16(y), or int8 rint(y / (max|y| / 127)) + scale,
//                    or E4M3FN(y / (max|y| / 448)) + scale (codes saturate
//                    at +-127 / +-448 where a subnormal scale lets the
//                    quotient pass them)
//   k_cache[row]   = bf16(kr)
//
// Design (HBM-bound; nothing here is a dense contraction, so no MFMA):
//   * one wavefront owns TPW whole token rows; the 64 lanes split into TPW
//     groups of 64/TPW lanes, one group per row;
//   * a group reads its kv row with coalesced 16-byte loads: lane l holds the
//     8-element chunks l, l + 64/TPW, ... so every load instruction covers a
//     contiguous stretch of the row, and writes the ckv row back the same way;
//   * the square sum runs in a fixed order (per-chunk partials folded in
//     halves: in-lane first, then xor shuffles), so the result is the same for
//     every TPW (the order stated in include/kvrc.h);
//   * the RoPE half is spread so that each lane produces 64/(64/TPW)
//     consecutive outputs: one contiguous store per lane;
//   * sqrt is correctly rounded and x/rms, amax/127, y/scale are correctly
//     rounded divisions (IEEE, or the shared-divisor form of
//     device_common.hpp on its domain), so the outputs and the int8 and
//     E4M3FN codes are bit-identical to the float32 definition.
//
// The specialised kernel handles Dv = 512, Dk = 64 (the DeepSeek-V3 latent
// key row); every other multiple-of-8 shape takes the generic kernel (one
// token per wavefront, loops over chunks).
#include "device_common.hpp"
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

#ifndef KVRC_WG_THREADS
#define KVRC_WG_THREADS 256                // 4 wavefronts per workgroup
#endif
constexpr int kThreads = KVRC_WG_THREADS;
constexpr int kWaves = kThreads / 64;

// n / d for a divisor fixed per launch (see make_udiv).
__device__ __forceinline__ uint32_t udiv(uint32_t n, UDiv d)
{
    if (d.shift == 0)
        return n;                                        // divisor 1
    const uint32_t t = __umulhi(n, d.magic);
    return (t + ((n - t) >> 1)) >> (d.shift - 1);
}

// Position of token t's entry in the index array (T and S fit 32 bits).
__device__ __forceinline__ int64_t index_pos(const NormRopeCacheArgs &a, int64_t t)
{
    if (a.chunks_per_seq == 0)
        return t;
    const uint32_t b = udiv((uint32_t)t, a.div_s), s = (uint32_t)t - b * (uint32_t)a.S;
    return (int64_t)b * a.chunks_per_seq + udiv(s, a.div_bs);
}

// Destination row of token t with index value v, or -1 (skip). Counts
// invalid index values.
__device__ __forceinline__ int64_t dest_row(const NormRopeCacheArgs &a, int64_t v, int64_t t,
                                            bool leader)
{
    if (v >= 0 && v < a.limit) {
        if (a.rows_per_batch)
            return (int64_t)udiv((uint32_t)t, a.div_s) * a.rows_per_batch + v;
        if (a.chunks_per_seq) {
            const uint32_t s = (uint32_t)t - udiv((uint32_t)t, a.div_s) * (uint32_t)a.S;
            const uint32_t bs = (uint32_t)a.block_size;
            const uint64_t blk = (uint64_t)v <= 0xffffffffull
                ? (uint64_t)udiv((uint32_t)v, a.div_bs) : (uint64_t)v / bs;
            return (int64_t)(blk * bs + (s - udiv(s, a.div_bs) * bs));
        }
        return v;
    }
    if (v != -1 && leader && a.err)
        atomicAdd(a.err, 1);
    return -1;
}

// RoPE output o of a row (0 <= o < dk): pair i = o mod dk/2.
__device__ __forceinline__ float rope_out(float xe, float xo, float c, float s, bool upper)
{
    // lower half: x[2i]*c - x[2i+1]*s ; upper half: x[2i+1]*c + x[2i]*s
    const float p1 = (upper ? xo : xe) * c;
    const float p2 = (upper ? xe : xo) * s;
    return upper ? p1 + p2 : p1 - p2;
}

// Cache rows are written with sc1 (device scope) stores when the cache fits
// a buffer descriptor (BUF: each cache smaller than 4 GiB): the rows are
// written through the XCD's L2 instead of being left dirty there, which on
// MI355X spares the write-back of up to the L2's capacity of dirty lines at
// the end of the kernel (measured faster than the default policy and than
// non-temporal stores). The descriptor covers exactly the cache, so the
// hardware also drops any store outside it. Larger caches use plain global
// stores.
#ifndef KVRC_STORE_AUX
#define KVRC_STORE_AUX 16
#endif

template <bool BUF>
class CacheWriter {
  public:
    __device__ CacheWriter(void *cache, int64_t bytes) : base_(static_cast<unsigned char *>(cache))
    {
        if constexpr (BUF)
            rsrc_ = __builtin_amdgcn_make_buffer_rsrc(cache, 0, (int)(uint32_t)bytes, kWord3);
    }
    template <typename T>
    __device__ void store(int64_t off, T v) const
    {
        if constexpr (BUF)
            buffer_store(rsrc_, (int)(uint32_t)off, v);
        else
            *reinterpret_cast<T *>(base_ + off) = v;
    }

  private:
    // Word 3 of a raw (untyped) gfx9 buffer descriptor: 32-bit data format.
    static constexpr int kWord3 = 0x00020000;
    static __device__ void buffer_store(__amdgpu_buffer_rsrc_t r, int off, u32x4 v)
    {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, KVRC_STORE_AUX);
    }
    static __device__ void buffer_store(__amdgpu_buffer_rsrc_t r, int off, u32x2 v)
    {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, KVRC_STORE_AUX);
    }
    static __device__ void buffer_store(__amdgpu_buffer_rsrc_t r, int off, uint32_t v)
    {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, KVRC_STORE_AUX);
    }
    static __device__ void buffer_store(__amdgpu_buffer_rsrc_t r, int off, uint16_t v)
    {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, KVRC_STORE_AUX);
    }
    unsigned char *base_;
    __amdgpu_buffer_rsrc_t rsrc_;
};

// ---------------------------------------------------------------------------
// Dv = 512, Dk = 64: TPW token rows per wavefront.
// ---------------------------------------------------------------------------
template <int TPW, int CKV, bool BUF, int NT>
__global__ __launch_bounds__(NT) void norm_rope_cache_d576(NormRopeCacheArgs a)
{
    constexpr int DV = 512, DK = 64, D = DV + DK;
    constexpr int LPT = 64 / TPW;         // lanes per token row
    constexpr int NCH = DV / 8 / LPT;     // 16-byte chunks of the norm half per lane
    constexpr int ROUT = DK / LPT;        // RoPE outputs per lane

    const int lane = threadIdx.x & 63;
    const int l = lane % LPT;
    const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    const int64_t t = wave * TPW + lane / LPT;
    if (t >= a.T)
        return;
    // The token's inputs do not depend on its index value, so every load is
    // issued before the index is examined and their latencies overlap; the
    // stores alone are conditional (a skipped token's reads are wasted).
    const int64_t v = a.index[index_pos(a, t)];

    // ---- loads: norm half, gamma, RoPE half, cos/sin -----------------------
    const uint16_t *xr = a.kv + t * D;
    uint4 xq[NCH], gq[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c = l + LPT * j;
        xq[j] = to_uint4(stream_load<u32x4>(xr + 8 * c));
        gq[j] = *reinterpret_cast<const uint4 *>(a.gamma + 8 * c);
    }
    const int o0 = l * ROUT;              // first RoPE output of this lane
    const bool upper = o0 >= DK / 2;
    const int i0 = o0 & (DK / 2 - 1);     // first pair index
    float xe[ROUT], xo[ROUT], cv[ROUT], sv[ROUT];
    {
        const uint16_t *pr = xr + DV + 2 * i0;
        const uint16_t *cr = a.cos + t * DK + o0;
        const uint16_t *sr = a.sin + t * DK + o0;
        if constexpr (ROUT == 1) {
            const uint32_t w = stream_load<uint32_t>(pr);
            xe[0] = bf16_lo(w); xo[0] = bf16_hi(w);
            cv[0] = __uint_as_float((uint32_t)stream_load<uint16_t>(cr) << 16);
            sv[0] = __uint_as_float((uint32_t)stream_load<uint16_t>(sr) << 16);
        } else if constexpr (ROUT == 2) {
            const uint2 w = to_uint2(stream_load<u32x2>(pr));
            const uint32_t cw = stream_load<uint32_t>(cr);
            const uint32_t sw = stream_load<uint32_t>(sr);
            xe[0] = bf16_lo(w.x); xo[0] = bf16_hi(w.x);
            xe[1] = bf16_lo(w.y); xo[1] = bf16_hi(w.y);
            cv[0] = bf16_lo(cw); cv[1] = bf16_hi(cw);
            sv[0] = bf16_lo(sw); sv[1] = bf16_hi(sw);
        } else {
            static_assert(ROUT == 4, "TPW must be 1, 2 or 4");
            const uint4 w = to_uint4(stream_load<u32x4>(pr));
            const uint2 cw = to_uint2(stream_load<u32x2>(cr));
            const uint2 sw = to_uint2(stream_load<u32x2>(sr));
            xe[0] = bf16_lo(w.x); xo[0] = bf16_hi(w.x);
            xe[1] = bf16_lo(w.y); xo[1] = bf16_hi(w.y);
            xe[2] = bf16_lo(w.z); xo[2] = bf16_hi(w.z);
            xe[3] = bf16_lo(w.w); xo[3] = bf16_hi(w.w);
            cv[0] = bf16_lo(cw.x); cv[1] = bf16_hi(cw.x);
            cv[2] = bf16_lo(cw.y); cv[3] = bf16_hi(cw.y);
            sv[0] = bf16_lo(sw.x); sv[1] = bf16_hi(sw.x);
            sv[2] = bf16_lo(sw.y); sv[3] = bf16_hi(sw.y);
        }
    }

    const int64_t row = dest_row(a, v, t, l == 0);
    const bool write = row >= 0;

    // ---- RMSNorm: canonical square sum -----------------------------------
    float x[NCH][8];
    float part[NCH];
    uint32_t min_sq = 0xffffffffu;        // smallest square (bits) seen by this lane
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        unpack8(xq[j], x[j]);
        part[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sq = x[j][e] * x[j][e];
            part[j] = part[j] + sq;
            min_sq = min(min_sq, __float_as_uint(sq));
        }
    }
    // chunk l + LPT*j is partial (l + LPT*j) of 64; fold in halves in-lane
    // (w = 64 .. LPT) and then across the LPT lanes of the row.
#pragma unroll
    for (int w = NCH; w > 1; w /= 2)
#pragma unroll
        for (int k = 0; k < w / 2; ++k)
            part[k] = part[k] + part[k + w / 2];
    const float ss = fold_sum<LPT>(part[0]);
    const float ms = ss / (float)DV;
    const float rms = sqrtf(ms + a.eps);

    // q = x / rms: shared-divisor division when rms and every |x| of this lane
    // are inside its domain (|x| >= 2^-60 and |x| <= sqrt(Dv)*rms), else IEEE.
    float y[NCH][8];
    if (fast_div_divisor_ok(rms) && min_sq >= kMinSquareBits) {
        const float rr = rcp_rn(rms);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            float g[8];
            unpack8(gq[j], g);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                y[j][e] = div_rn_shared(x[j][e], rms, rr) * g[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            float g[8];
            unpack8(gq[j], g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float q = x[j][e] / rms;
                y[j][e] = q * g[e];
            }
        }
    }

    if constexpr (CKV == kCkvInt8) {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(y[j][e]));
        amax = fold_max<LPT>(amax);
        const float scale = row_scale(amax, 127.0f);
        // code = rint(RN(y / scale)), half to even. In the shared-divisor
        // domain of scale, with rs = RN(1/scale) and P = y * rs (exact):
        //   |P - y/scale| and |RN(y/scale) - y/scale| are both below
        //   2^-24 * 127.0001 < 2^-17, so |P - RN(y/scale)| < 2^-16;
        //   RN(P + 1.5*2^23) = 1.5*2^23 + rint(P) (one fma; the low byte of
        //   its bits is the int8 code of rint(P));
        //   rint(P) and rint(RN(y/scale)) differ only if a half-integer h lies
        //   within 2^-16 of P. f = RN(P + 384) lies in (256, 512) with ulp
        //   2^-15, so its 15 low mantissa bits are frac(P) in units of 2^-15
        //   and |f - 384 - h| < 2^-15 forces them to 0x4000 exactly.
        // Lanes with an element whose f has low bits 0x3fff..0x4001 redo their
        // quotients exactly (elements with |y| below the shared-divisor
        // dividend range have |quotient| < 2^-4 and code 0 either way).
        uint32_t cb[NCH][8];
        if (fast_div_divisor_ok(scale)) {
            const float rs = rcp_rn(scale);
            // smallest (low 15 bits of f + 0x4001) << 17 over the lane: at most
            // 2 << 17 exactly when some low bits are 0x3fff, 0x4000 or 0x4001
            uint32_t dmin = 0xffffffffu;
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    cb[j][e] = __float_as_uint(__builtin_fmaf(y[j][e], rs, kRoundMagic));
                    const uint32_t f = __float_as_uint(__builtin_fmaf(y[j][e], rs, 384.0f));
                    dmin = min(dmin, (f + 0x4001u) << 17);
                }
            if (dmin <= (2u << 17)) {
#pragma unroll
                for (int j = 0; j < NCH; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        cb[j][e] = __float_as_uint(div_rn_shared(y[j][e], scale, rs) + kRoundMagic);
            }
        } else {
            // scale 0, tiny or huge: IEEE division. A scale rounded to a
            // float32 subnormal can push |y / scale| past 127: saturate.
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float qv = scale == 0.0f ? 0.0f : y[j][e] / scale;
                    cb[j][e] = __float_as_uint(__builtin_amdgcn_fmed3f(qv, -127.0f, 127.0f) +
                                               kRoundMagic);
                }
        }
        if (write) {
            const CacheWriter<BUF> dst(a.ckv_cache, a.cache_rows * DV);
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                dst.store(row * DV + 8 * (l + LPT * j), pack_low_bytes8(cb[j]));
            if (l == 0)
                a.ckv_scale[row] = scale;
        }
    } else if constexpr (CKV == kCkvFp8) {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(y[j][e]));
        amax = fold_max<LPT>(amax);
        const float scale = row_scale(amax, kE4m3Max);
        // The code is that of Q = RN(y / scale). In the shared-divisor domain
        // of scale, t = RN(y * RN(1/scale)) is within |Q| * (2^-23 + 2^-48)
        // of y / scale, so t and Q lie less than 2.5 ulps apart; the rounding
        // to E4M3FN is monotonic, so both get the same code unless a midpoint
        // between two E4M3FN values lies within 2.5 ulps of t. Lanes holding
        // such an element, or one below 2^-6 (the E4M3FN subnormal range,
        // whose midpoints have other bit patterns), redo the quotients
        // exactly. Everywhere here |t| and |Q| stay below 448 * (1 + 2^-22),
        // inside the conversion's range.
        float q[NCH][8];
        if (fast_div_divisor_ok(scale)) {
            const float rs = rcp_rn(scale);
            uint32_t kmin = 0xffffffffu;  // smallest midpoint key of the lane
            float tmin = __builtin_inff(); // smallest |t| of the lane
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = y[j][e] * rs;
                    q[j][e] = t;
                    kmin = min(kmin, e4m3_midpoint_key(t));
                    tmin = fminf(tmin, fabsf(t));
                }
            if (kmin < kE4m3NearKey || tmin < 0x1p-6f) {
                bool tiny = false;        // shared-divisor domain: |y| >= 2^-64
#pragma unroll
                for (int j = 0; j < NCH; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        tiny |= fabsf(y[j][e]) < kFastDivDividendLo;
                if (!tiny) {
#pragma unroll
                    for (int j = 0; j < NCH; ++j)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            q[j][e] = div_rn_shared(y[j][e], scale, rs);
                } else {
#pragma unroll
                    for (int j = 0; j < NCH; ++j)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            q[j][e] = y[j][e] / scale;
                }
            }
        } else {
            // scale 0 (an all-zero row: codes 0), tiny or huge: IEEE division;
            // a scale rounded to a float32 denormal can push |Q| past 448.
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    q[j][e] = scale == 0.0f ? 0.0f : e4m3_clamp(y[j][e] / scale);
        }
        if (write) {
            const CacheWriter<BUF> dst(a.ckv_cache, a.cache_rows * DV);
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                dst.store(row * DV + 8 * (l + LPT * j), e4m3_pack8(q[j]));
            if (l == 0)
                a.ckv_scale[row] = scale;
        }
    } else if (write) {
        const CacheWriter<BUF> dst(a.ckv_cache, a.cache_rows * DV * 2);
#pragma unroll
        for (int j = 0; j < NCH; ++j)
            dst.store((row * DV + 8 * (l + LPT * j)) * 2, to_u32x4(pack8(y[j])));
    }

    // ---- RoPE ---------------------------------------------------------------
    float kr[ROUT];
#pragma unroll
    for (int r = 0; r < ROUT; ++r)
        kr[r] = rope_out(xe[r], xo[r], cv[r], sv[r], upper);
    if (!write)
        return;
    const CacheWriter<BUF> kdst(a.k_cache, a.cache_rows * DK * 2);
    const int64_t koff = (row * DK + o0) * 2;
    if constexpr (ROUT == 1)
        kdst.store(koff, (uint16_t)(pack_bf16x2(kr[0], 0.0f) & 0xffffu));
    else if constexpr (ROUT == 2)
        kdst.store(koff, pack_bf16x2(kr[0], kr[1]));
    else
        kdst.store(koff, u32x2{pack_bf16x2(kr[0], kr[1]), pack_bf16x2(kr[2], kr[3])});
}

// ---------------------------------------------------------------------------
// Any Dv, Dk that are multiples of 8: one token per wavefront.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void norm_rope_cache_generic(NormRopeCacheArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= a.T)
        return;
    const int64_t row = dest_row(a, a.index[index_pos(a, t)], t, lane == 0);
    if (row < 0)
        return;
    const int64_t Dv = a.Dv, Dk = a.Dk, D = Dv + Dk;
    const uint16_t *xr = a.kv + t * D;
    const int64_t nch = Dv / 8;

    // partial `lane` accumulates chunks lane, lane + 64, ... in order
    float part = 0.0f;
    for (int64_t c = lane; c < nch; c += 64) {
        float x[8];
        unpack8(*reinterpret_cast<const uint4 *>(xr + 8 * c), x);
        part = chunk_sumsq(x, part);
    }
    const float ss = fold_sum<64>(part);
    const float ms = ss / (float)Dv;
    const float rms = sqrtf(ms + a.eps);

    if (a.ckv != kCkvBf16) {
        const bool fp8 = a.ckv == kCkvFp8;
        float amax = 0.0f;
        for (int64_t c = lane; c < nch; c += 64) {
            float x[8], g[8];
            unpack8(*reinterpret_cast<const uint4 *>(xr + 8 * c), x);
            unpack8(*reinterpret_cast<const uint4 *>(a.gamma + 8 * c), g);
            for (int e = 0; e < 8; ++e) {
                const float q = x[e] / rms;
                amax = fmaxf(amax, fabsf(q * g[e]));
            }
        }
        amax = fold_max<64>(amax);
        const float scale = amax / (fp8 ? kE4m3Max : 127.0f);
        uint8_t *dst = static_cast<uint8_t *>(a.ckv_cache) + row * Dv;
        for (int64_t c = lane; c < nch; c += 64) {
            float x[8], g[8], code[8];
            unpack8(*reinterpret_cast<const uint4 *>(xr + 8 * c), x);
            unpack8(*reinterpret_cast<const uint4 *>(a.gamma + 8 * c), g);
            for (int e = 0; e < 8; ++e) {
                const float q = x[e] / rms;
                const float yv = q * g[e];
                const float qs = scale == 0.0f ? 0.0f : yv / scale;
                code[e] = fp8 ? e4m3_clamp(qs) : rintf(__builtin_amdgcn_fmed3f(qs, -127.0f, 127.0f));
            }
            *reinterpret_cast<uint2 *>(dst + 8 * c) =
                fp8 ? to_uint2(e4m3_pack8(code)) : pack_codes8(code);
        }
        if (lane == 0)
            a.ckv_scale[row] = scale;
    } else {
        uint16_t *dst = static_cast<uint16_t *>(a.ckv_cache) + row * Dv;
        for (int64_t c = lane; c < nch; c += 64) {
            float x[8], g[8], yv[8];
            unpack8(*reinterpret_cast<const uint4 *>(xr + 8 * c), x);
            unpack8(*reinterpret_cast<const uint4 *>(a.gamma + 8 * c), g);
            for (int e = 0; e < 8; ++e) {
                const float q = x[e] / rms;
                yv[e] = q * g[e];
            }
            *reinterpret_cast<uint4 *>(dst + 8 * c) = pack8(yv);
        }
    }

    const int64_t h = Dk / 2;
    for (int64_t o = lane; o < Dk; o += 64) {
        const bool upper = o >= h;
        const int64_t i = upper ? o - h : o;
        const uint32_t w = *reinterpret_cast<const uint32_t *>(xr + Dv + 2 * i);
        const float c = __uint_as_float((uint32_t)a.cos[t * Dk + o] << 16);
        const float s = __uint_as_float((uint32_t)a.sin[t * Dk + o] << 16);
        const float v = rope_out(bf16_lo(w), bf16_hi(w), c, s, upper);
        a.k_cache[row * Dk + o] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
}

template <int TPW, int CKV, int NT>
hipError_t launch_d576(const NormRopeCacheArgs &a, hipStream_t stream)
{
    const int64_t tokens_per_wg = (int64_t)(NT / 64) * TPW;
    const int64_t grid = (a.T + tokens_per_wg - 1) / tokens_per_wg;
    // Buffer descriptors hold 32-bit sizes and offsets: each cache must be
    // smaller than 4 GiB for the sc1 buffer stores.
    const int64_t rows = a.cache_rows;
    const bool buf = rows * 512 * (CKV == kCkvBf16 ? 2 : 1) <= (int64_t)UINT32_MAX &&
                     rows * 64 * 2 <= (int64_t)UINT32_MAX;
    if (buf)
        hipLaunchKernelGGL((norm_rope_cache_d576<TPW, CKV, true, NT>), dim3((uint32_t)grid),
                           dim3(NT), 0, stream, a);
    else
        hipLaunchKernelGGL((norm_rope_cache_d576<TPW, CKV, false, NT>), dim3((uint32_t)grid),
                           dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Rows per wavefront for the Dv = 512 / Dk = 64 kernel (measured best on
// MI355X: 2 for both; 4 rows per wavefront shares more per-row work but needs
// twice the registers, and 1 row halves the work per load instruction).
#ifndef KVRC_TPW_BF16
#define KVRC_TPW_BF16 2
#endif
#ifndef KVRC_TPW_INT8
#define KVRC_TPW_INT8 2
#endif
#ifndef KVRC_TPW_FP8
#define KVRC_TPW_FP8 2
#endif

// Up to this many tokens (a decode step) the chip is far from full: one row
// per wavefront in one-wavefront workgroups spreads the rows over the most
// compute units and shortens each wavefront's work (measured 2.74 -> 2.49 us
// per step for 256 rows).
constexpr int64_t kSmallBatchTokens = 2048;

hipError_t launch_norm_rope_cache(const NormRopeCacheArgs &a, hipStream_t stream)
{
    if (a.Dv == 512 && a.Dk == 64) {
        if (a.T <= kSmallBatchTokens) {
            switch (a.ckv) {
            case kCkvInt8: return launch_d576<1, kCkvInt8, 64>(a, stream);
            case kCkvFp8: return launch_d576<1, kCkvFp8, 64>(a, stream);
            default: return launch_d576<1, kCkvBf16, 64>(a, stream);
            }
        }
        switch (a.ckv) {
        case kCkvInt8: return launch_d576<KVRC_TPW_INT8, kCkvInt8, kThreads>(a, stream);
        case kCkvFp8: return launch_d576<KVRC_TPW_FP8, kCkvFp8, kThreads>(a, stream);
        default: return launch_d576<KVRC_TPW_BF16, kCkvBf16, kThreads>(a, stream);
        }
    }
    const int64_t grid = (a.T + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(norm_rope_cache_generic, dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvrc
