// QSAPrepare block keys for gfx950 (openvino.opset17.qsa_prepare: one key
// per complete key block = mean of the block's key_block_size raw keys,
// RMS-normalised with k_norm_weight and rotated with the RoPE of the block's
// first token; only blocks completed by the new tokens are computed).
//
// Work decomposition: one 256-thread workgroup per (sequence, new block),
// plus one workgroup per sequence that writes the carry state for the next
// call. The host cannot see key_length (it stays in device memory), so the
// grid is sized for the largest possible number of new blocks,
// floor((kbs-1+L)/kbs), and a workgroup whose block does not exist returns.
//
// Block mean: the block's rows are staged through LDS. All threads load
// 16-byte pieces of the rows at once (branch-free, so every load of a chunk
// is in flight together), write them to LDS, and then each thread adds its
// dimension pair down the rows in token order. The float32 sum therefore has
// the definition's order whatever the chunking of the token stream across
// calls (the only rows that come from the carried state are the first ones of
// the block that straddles it). Chunks of at most kStageBytes of rows keep the
// LDS footprint bounded for any key_block_size and Di.
// The mean then goes through LDS once more for the norm (canonical chunk
// layout of the square sum: 8 dims per chunk, partials folded in halves) and
// the RoPE of the trailing Dr dims.
#include "device_common.hpp"
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;                // 16-byte row pieces per thread per chunk
constexpr int kStageBytes = kVecPerThread * 16 * kThreads;    // 16 KiB of rows per chunk
constexpr int kRopePrefetch = 2;                // cos/sin/weight values per thread fetched early

// PPT: dimension pairs per thread, Di/2 <= 256*PPT (kept small so that the
// common Di = 128 uses few registers and every workgroup fits in one round).
template <int PPT>
__global__ __launch_bounds__(kThreads) void qsa_prepare_kernel(QsaArgs a, int64_t nb_max,
                                                               int64_t rows_per_chunk)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const uint32_t per = (uint32_t)(nb_max + 1);       // grid < 2^31
    const int64_t n = blockIdx.x / per;
    const int64_t j = blockIdx.x % per;
    const int64_t K = a.key_length[a.klc == 1 ? 0 : n];
    const int64_t kbs = a.kbs, Di = a.Di, L = a.L;
    if (K < L || K / kbs > a.Bcap) {
        if (j == 0 && tid == 0 && a.err)
            atomicAdd(a.err, 1);
        return;
    }
    const int64_t P = K - L;
    const int64_t r = P % kbs;
    const int64_t vec_per_row = Di / 8;
    const uint32_t vpr = (uint32_t)vec_per_row;       // <= 512: 32-bit index math

    if (j == nb_max) {
        // ---- carry state: tokens [t1, K) of the incomplete block ----------
        const int64_t r2 = K % kbs, t1 = K - r2;
        const int64_t total = r2 * vec_per_row;
        for (int64_t e0 = 0; e0 < total; e0 += (int64_t)kThreads * kVecPerThread) {
            u32x4 buf[kVecPerThread];
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k) {
                int64_t e = e0 + tid + (int64_t)kThreads * k;
                e = e < total ? e : total - 1;            // clamp: loads stay branch-free
                const uint32_t ue = (uint32_t)e;          // total <= (kbs-1) * 512 < 2^32
                const int64_t i = ue / vpr, c = ue % vpr;
                const int64_t tau = t1 + i;
                const uint16_t *src = tau < P
                    ? a.past_raw + (n * (kbs - 1) + (tau - (P - r))) * Di
                    : a.raw + (n * L + (tau - P)) * Di;
                buf[k] = *reinterpret_cast<const u32x4 *>(src + 8 * c);
            }
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k) {
                const int64_t e = e0 + tid + (int64_t)kThreads * k;
                if (e < total) {
                    const int64_t i = (uint32_t)e / vpr, c = (uint32_t)e % vpr;
                    *reinterpret_cast<u32x4 *>(a.next_raw + (n * (kbs - 1) + i) * Di + 8 * c) =
                        buf[k];
                }
            }
        }
        if (a.rope_cos && r2 > 0) {
            const int64_t Dr = a.Dr;
            for (int64_t d = tid; d < Dr; d += kThreads) {
                float c, s;
                if (t1 < P) {
                    c = a.past_rope[n * 2 * Dr + d];
                    s = a.past_rope[n * 2 * Dr + Dr + d];
                } else {
                    c = a.rope_cos[(n * L + (t1 - P)) * Dr + d];
                    s = a.rope_sin[(n * L + (t1 - P)) * Dr + d];
                }
                a.next_rope[n * 2 * Dr + d] = c;
                a.next_rope[n * 2 * Dr + Dr + d] = s;
            }
        }
        return;
    }

    const int64_t b = P / kbs + j;
    if (b >= K / kbs)
        return;
    const int64_t tau0 = b * kbs;                       // first token of the block
    // rows [0, np) of the block are carried rows 0.. (only when it straddles)
    const int64_t np = tau0 < P ? P - tau0 : 0;
    const uint16_t *past_base = a.past_raw + n * (kbs - 1) * Di;
    const uint16_t *new_base = a.raw + n * L * Di;      // new row i: token P + i

    // cos/sin of the block's first token (fetched right after the first
    // chunk of rows, so that the two sets of loads are in flight together).
    const int64_t Dr = a.rope_cos ? a.Dr : 0;
    const float *cr = nullptr, *sr = nullptr;
    if (Dr) {
        if (tau0 < P) {
            cr = a.past_rope + n * 2 * Dr;
            sr = cr + Dr;
        } else {
            cr = a.rope_cos + (n * L + (tau0 - P)) * Dr;
            sr = a.rope_sin + (n * L + (tau0 - P)) * Dr;
        }
    }

    uint16_t *stage = reinterpret_cast<uint16_t *>(smem);
    float *m = reinterpret_cast<float *>(smem + kStageBytes);
    float *z = m + Di;

    // ---- block mean: float32 sum down the rows, in token order ------------
    const int64_t npairs = Di / 2;
    float acc[2 * PPT];
#pragma unroll
    for (int k = 0; k < 2 * PPT; ++k)
        acc[k] = 0.0f;
    u32x4 buf[kVecPerThread];
    // Issue the loads of rows [row0, row0 + rows) into buf (branch-free).
    auto load_rows = [&](int64_t row0, int64_t rows) {
        const uint32_t total = (uint32_t)(rows * vec_per_row);    // <= 1024
#pragma unroll
        for (int k = 0; k < kVecPerThread; ++k) {
            uint32_t e = (uint32_t)(tid + kThreads * k);
            e = e < total ? e : total - 1;
            const int64_t i = row0 + e / vpr, c = e % vpr;
            const uint16_t *src = i < np ? past_base + i * Di : new_base + (tau0 + i - P) * Di;
            buf[k] = stream_load<u32x4>(src + 8 * c);
        }
    };
    // Stage buf through LDS and add the rows to the running sums in order.
    auto add_rows = [&](int64_t rows) {
        const int64_t total = rows * vec_per_row;
        __syncthreads();                                 // previous chunk consumed
#pragma unroll
        for (int k = 0; k < kVecPerThread; ++k) {
            const int64_t e = tid + (int64_t)kThreads * k;
            if (e < total)
                *reinterpret_cast<u32x4 *>(stage + 8 * e) = buf[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int64_t p = tid + (int64_t)kThreads * k;
            if (p < npairs) {
                const uint32_t *col = reinterpret_cast<const uint32_t *>(stage) + p;
                float s0 = acc[2 * k], s1 = acc[2 * k + 1];
#pragma unroll 16
                for (int64_t i = 0; i < rows; ++i) {
                    const uint32_t w = col[i * npairs];
                    s0 = s0 + bf16_lo(w);
                    s1 = s1 + bf16_hi(w);
                }
                acc[2 * k] = s0;
                acc[2 * k + 1] = s1;
            }
        }
    };

    const int64_t rows0 = kbs < rows_per_chunk ? kbs : rows_per_chunk;
    load_rows(0, rows0);
    float cs_pre[kRopePrefetch], sn_pre[kRopePrefetch], w_pre[kRopePrefetch];
#pragma unroll
    for (int k = 0; k < kRopePrefetch; ++k) {
        const int64_t o = tid + (int64_t)kThreads * k;
        cs_pre[k] = o < Dr ? cr[o] : 0.0f;
        sn_pre[k] = o < Dr ? sr[o] : 0.0f;
        w_pre[k] = a.weight && o < Di ? __uint_as_float((uint32_t)a.weight[o] << 16) : 0.0f;
    }
    add_rows(rows0);
    for (int64_t row0 = rows0; row0 < kbs; row0 += rows_per_chunk) {
        const int64_t rows = kbs - row0 < rows_per_chunk ? kbs - row0 : rows_per_chunk;
        load_rows(row0, rows);
        add_rows(rows);
    }
    const float fk = (float)kbs;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int64_t p = tid + (int64_t)kThreads * k;
        if (p < npairs) {
            m[2 * p] = acc[2 * k] / fk;
            m[2 * p + 1] = acc[2 * k + 1] / fk;
        }
    }
    __syncthreads();

    // ---- RMS normalisation over Di (canonical square sum, wavefront 0) ----
    const int64_t nch = Di / 8;
    float *rms_slot = z + Di;                           // one float of LDS
    if (a.weight) {
        if (tid < 64) {
            float part = 0.0f;
            for (int64_t c = tid; c < nch; c += 64) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = m[8 * c + e];
                part = chunk_sumsq(x, part);
            }
            const float ss = fold_sum<64>(part);
            if (tid == 0)
                *rms_slot = sqrtf(ss / (float)Di + a.eps);
        }
        __syncthreads();
        const float rms = *rms_slot;
#pragma unroll
        for (int k = 0; k < kRopePrefetch; ++k) {
            const int64_t d = tid + (int64_t)kThreads * k;
            if (d < Di)
                z[d] = (m[d] / rms) * w_pre[k];
        }
        for (int64_t d = tid + (int64_t)kThreads * kRopePrefetch; d < Di; d += kThreads) {
            const float q = m[d] / rms;
            z[d] = q * __uint_as_float((uint32_t)a.weight[d] << 16);
        }
    } else {
        for (int64_t d = tid; d < Di; d += kThreads)
            z[d] = m[d];
    }
    __syncthreads();

    // ---- RoPE of the trailing Dr dims with the first token's cos/sin -----
    // The rotated values go to the (no longer needed) mean buffer m[0, Dr).
    const int64_t base = Di - Dr;
    if (Dr) {
        const int64_t h = Dr / 2;
#pragma unroll
        for (int k = 0; k < kRopePrefetch; ++k) {
            const int64_t o = tid + (int64_t)kThreads * k;
            if (o < Dr) {
                const bool upper = o >= h;
                const int64_t i = upper ? o - h : o;
                const float xe = z[base + 2 * i], xo = z[base + 2 * i + 1];
                const float p1 = (upper ? xo : xe) * cs_pre[k];
                const float p2 = (upper ? xe : xo) * sn_pre[k];
                m[o] = upper ? p1 + p2 : p1 - p2;
            }
        }
        for (int64_t o = tid + (int64_t)kThreads * kRopePrefetch; o < Dr; o += kThreads) {
            const bool upper = o >= h;
            const int64_t i = upper ? o - h : o;
            const float xe = z[base + 2 * i], xo = z[base + 2 * i + 1];
            const float p1 = (upper ? xo : xe) * cr[o];
            const float p2 = (upper ? xe : xo) * sr[o];
            m[o] = upper ? p1 + p2 : p1 - p2;
        }
        __syncthreads();
    }

    // ---- store bf16 key ----------------------------------------------------
    uint16_t *dst = a.block_keys + (n * a.Bcap + b) * Di;
    for (int64_t c = tid; c < nch; c += kThreads) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t d = 8 * c + e;
            v[e] = d < base ? z[d] : m[d - base];
        }
        *reinterpret_cast<u32x4 *>(dst + 8 * c) = to_u32x4(pack8(v));
    }
}

// ---------------------------------------------------------------------------
// Di = 128 and blocks of at most 64 rows: one wavefront per (sequence, new
// block), lane l owning the dimension pair (2 l, 2 l + 1) of the key. The
// block's rows go straight from memory into LDS, four rows per 1 KiB load
// (16 loads, up to 10 of them in flight: no staging registers, no LDS
// stores); as each load lands, the lanes read their pair from its four rows
// and add them to their running sums in token order. The norm's chunk c
// (dims 8 c .. 8 c + 7) lies on lanes 4 c .. 4 c + 3; its square sum is
// taken in element order, then the 16 chunk partials are folded in halves
// (c + 8, + 4, + 2, + 1): the same operations in the same order as the
// general kernel, so the keys are bit-identical.
// ---------------------------------------------------------------------------
constexpr int kWaveDi = 128;
constexpr int kWaveMaxRows = 64;
constexpr int kRowLoads = kWaveMaxRows / 4;     // 1 KiB loads: four 256-byte rows each
constexpr int kCpolNt = 2;                      // cache policy of the row loads: non-temporal

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most n vector memory loads of the
// wavefront are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; the
// other counters at their maxima, i.e. not waited for)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// At most kRowWindow of a block's 16 row loads are in flight at once:
// issuing all 16 together was slower (6.57 against 6.46 us per call on the
// 32 x 2048-token workload; a probe of the bare row reads: 4.97 against 4.62
// us with 6 in flight), the memory system serving a steady stream of
// requests better than one burst from every wavefront.
constexpr int kRowWindow = 10;

// Adds rows 4 K .. 4 K + 3 of the staged block (row i at stage[64 i], one
// dimension pair per lane) to the running sums once the K-th of the NK row
// loads has landed, issues load K + W into the freed window slot, then
// recurses to the next four rows. Loads complete in issue order and no other
// load is issued after the first row load, so the K-th has landed when at
// most min(NK - K, W) - 1 loads are outstanding. Full: all 4 NK rows belong
// to the block; otherwise rows i >= kbs add +0 (they hold a repeat of the
// last row). src(k) is lane's source address for load k.
template <int K, int NK, int W, bool Full>
struct RowWindowSum {
    template <typename Src>
    static __device__ __forceinline__ void run(uint32_t *stage, int lane, int64_t kbs, float &sum0,
                                               float &sum1, const Src &src)
    {
        constexpr int pending = NK - K < W ? NK - K : W;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(pending - 1));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = 4 * K + t;
            const uint32_t raw = stage[i * 64 + lane];
            const uint32_t v = Full || i < kbs ? raw : 0u;
            sum0 = sum0 + bf16_lo(v);
            sum1 = sum1 + bf16_hi(v);
        }
        if constexpr (K + W < NK) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_global_load_lds(src(K + W), (lds_void *)(stage + 256 * (K + W)), 16, 0,
                                             kCpolNt);
        }
        RowWindowSum<K + 1, NK, W, Full>::run(stage, lane, kbs, sum0, sum1, src);
    }
};
template <int NK, int W, bool Full>
struct RowWindowSum<NK, NK, W, Full> {
    template <typename Src>
    static __device__ __forceinline__ void run(uint32_t *, int, int64_t, float &, float &,
                                               const Src &)
    {
    }
};

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Work items are laid out XCD by XCD: workgroup g runs item
// (g mod 8) * per_xcd + g / 8 (round-robin dispatch puts workgroup g on XCD
// g mod 8), so each XCD takes a contiguous run of (sequence, block) items
// and touches one contiguous stretch of the raw keys (an eighth of the
// sequences) instead of a slice of every sequence: fewer pages per XCD's
// address translation cache and its L2 (measured 7.24 -> 7.11 us per call
// on the 32 x 2048-token workload).
constexpr uint32_t kXcds = 8;

__global__ __launch_bounds__(64) void qsa_prepare_wave_kernel(QsaArgs a, int64_t nb_max,
                                                              uint32_t per_xcd, uint32_t items)
{
    constexpr int64_t Di = kWaveDi;
    constexpr int kPairs = kWaveDi / 2;              // = 64 lanes
    const int lane = threadIdx.x;
    const uint32_t item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (item >= items)
        return;
    const uint32_t per = (uint32_t)(nb_max + 1);
    const int64_t n = item / per;
    const int64_t j = item % per;
    const int64_t K = a.key_length[a.klc == 1 ? 0 : n];
    const int64_t kbs = a.kbs, L = a.L;
    if (K < L || K / kbs > a.Bcap) {
        if (j == 0 && lane == 0 && a.err)
            atomicAdd(a.err, 1);
        return;
    }
    const int64_t P = K - L;
    const int64_t r = P % kbs;
    const int64_t Dr = a.rope_cos ? a.Dr : 0;

    if (j == nb_max) {
        // ---- carry state: tokens [t1, K) of the incomplete block ----------
        // At most kbs - 1 <= 63 rows of 16 pieces of 16 bytes: lane l takes
        // pieces l + 64 k (k < 16), indices past the end repeating the last
        // piece, and the rope row's values d = l, l + 64 (Dr <= 128). Every
        // load is issued before the first store: one memory round trip.
        const int64_t r2 = K % kbs, t1 = K - r2;
        if (r2 == 0)
            return;
        const int total = (int)r2 * 16;
        u32x4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = min(lane + 64 * k, total - 1);
            const int64_t tau = t1 + e / 16;
            const uint16_t *src = tau < P
                ? a.past_raw + (n * (kbs - 1) + (tau - (P - r))) * Di
                : a.raw + (n * L + (tau - P)) * Di;
            v[k] = *reinterpret_cast<const u32x4 *>(src + 8 * (e % 16));
        }
        float cv[2] = {0.0f, 0.0f}, sv[2] = {0.0f, 0.0f};
        if (Dr) {
            const float *cr, *sr;
            if (t1 < P) {
                cr = a.past_rope + n * 2 * Dr;
                sr = cr + Dr;
            } else {
                cr = a.rope_cos + (n * L + (t1 - P)) * Dr;
                sr = a.rope_sin + (n * L + (t1 - P)) * Dr;
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int d = lane + 64 * k;
                if (d < Dr) {
                    cv[k] = cr[d];
                    sv[k] = sr[d];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = min(lane + 64 * k, total - 1);
            *reinterpret_cast<u32x4 *>(a.next_raw + (n * (kbs - 1) + e / 16) * Di + 8 * (e % 16)) = v[k];
        }
        if (Dr) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int d = lane + 64 * k;
                if (d < Dr) {
                    a.next_rope[n * 2 * Dr + d] = cv[k];
                    a.next_rope[n * 2 * Dr + Dr + d] = sv[k];
                }
            }
        }
        return;
    }

    const int64_t b = P / kbs + j;
    if (b >= K / kbs)
        return;
    const int64_t tau0 = b * kbs;                       // first token of the block
    const int64_t np = tau0 < P ? P - tau0 : 0;         // rows taken from the carried state
    // this lane's outputs: dims d0 = 2 lane, d1 = d0 + 1; the RoPE covers
    // dims [base, 128), output o = d - base. Its cos/sin and weight values are
    // requested before the rows: no other load may be issued once the row
    // loads begin, whose completion is tracked by count below.
    const int64_t base = Di - Dr;
    const int d0 = 2 * lane;
    const bool rot = Dr && d0 >= base;
    float c0 = 0.0f, c1 = 0.0f, s0 = 0.0f, s1 = 0.0f;
    if (rot) {
        const int64_t o0 = d0 - base;
        const float *cr, *sr;
        if (tau0 < P) {
            cr = a.past_rope + n * 2 * Dr;
            sr = cr + Dr;
        } else {
            cr = a.rope_cos + (n * L + (tau0 - P)) * Dr;
            sr = a.rope_sin + (n * L + (tau0 - P)) * Dr;
        }
        c0 = cr[o0]; c1 = cr[o0 + 1];
        s0 = sr[o0]; s1 = sr[o0 + 1];
    }
    const uint32_t gw = a.weight ? *reinterpret_cast<const uint32_t *>(a.weight + d0) : 0u;

    // ---- the block's rows straight into LDS: load k brings rows 4 k .. 4 k + 3
    // (lane l: row 4 k + l / 16, 16-byte piece l % 16; the load writes lane l's
    // 16 bytes at byte 16 l of its 1 KiB, so row i lands at stage[64 i]).
    // Rows past kbs repeat the last row, so all 16 loads are always issued ---
    __shared__ __align__(16) uint32_t stage[kWaveMaxRows * kPairs];
    const int piece = lane & 15, sub = lane >> 4;
    const uint16_t *pastb = a.past_raw + n * (kbs - 1) * Di + 8 * piece;
    const uint16_t *rawb = a.raw + n * L * Di + 8 * piece;     // + (token - P) rows
    auto row_src = [&](int k) __attribute__((always_inline)) {
        const int64_t i = 4 * k + sub;
        const int64_t ii = i < kbs ? i : kbs - 1;
        return ii < np ? pastb + ii * Di : rawb + (tau0 + ii - P) * Di;
    };
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < kRowWindow; ++k)
        __builtin_amdgcn_global_load_lds(row_src(k), (lds_void *)(stage + 256 * k), 16, 0, kCpolNt);

    // ---- block mean: float32 sum down the rows in token order, four rows
    // at a time as their load lands (a sum that starts at +0 is never -0, so
    // the +0 terms past kbs leave it unchanged) ------------------------------
    float sum0 = 0.0f, sum1 = 0.0f;
    if (kbs == kWaveMaxRows)
        RowWindowSum<0, kRowLoads, kRowWindow, true>::run(stage, lane, kbs, sum0, sum1, row_src);
    else
        RowWindowSum<0, kRowLoads, kRowWindow, false>::run(stage, lane, kbs, sum0, sum1, row_src);
    const float fk = (float)kbs;
    const float m0 = sum0 / fk, m1 = sum1 / fk;

    // ---- RMS normalisation ------------------------------------------------
    float z0 = m0, z1 = m1;
    if (a.weight) {
        // chunk lane / 4: its 8 elements from the 4 lanes of the quad
        float x[8];
        x[0] = dpp_f<0x00>(m0); x[1] = dpp_f<0x00>(m1);     // quad_perm [0,0,0,0]
        x[2] = dpp_f<0x55>(m0); x[3] = dpp_f<0x55>(m1);     // [1,1,1,1]
        x[4] = dpp_f<0xAA>(m0); x[5] = dpp_f<0xAA>(m1);     // [2,2,2,2]
        x[6] = dpp_f<0xFF>(m0); x[7] = dpp_f<0xFF>(m1);     // [3,3,3,3]
        const float part = chunk_sumsq(x, 0.0f);
        float pc[16];
#pragma unroll
        for (int c = 0; c < 16; ++c)
            pc[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), 4 * c));
#pragma unroll
        for (int wdt = 16; wdt > 1; wdt /= 2)
#pragma unroll
            for (int c = 0; c < wdt / 2; ++c)
                pc[c] = pc[c] + pc[c + wdt / 2];
        const float rms = sqrtf(pc[0] / (float)Di + a.eps);
        z0 = (m0 / rms) * bf16_lo(gw);
        z1 = (m1 / rms) * bf16_hi(gw);
    }

    // ---- RoPE of the trailing Dr dims: output o takes the pair (2 i, 2 i + 1)
    // of the rotated part, i = o mod Dr / 2, held by lane base / 2 + i -------
    float y0 = z0, y1 = z1;
    if (Dr) {
        const int64_t h = Dr / 2;
        const int64_t o0 = d0 - base, o1 = o0 + 1;
        const bool up0 = o0 >= h, up1 = o1 >= h;
        const int src0 = rot ? (int)(base / 2 + (up0 ? o0 - h : o0)) : lane;
        const int src1 = rot ? (int)(base / 2 + (up1 ? o1 - h : o1)) : lane;
        const float xe0 = __shfl(z0, src0, 64), xo0 = __shfl(z1, src0, 64);
        const float xe1 = __shfl(z0, src1, 64), xo1 = __shfl(z1, src1, 64);
        if (rot) {
            const float p10 = (up0 ? xo0 : xe0) * c0, p20 = (up0 ? xe0 : xo0) * s0;
            const float p11 = (up1 ? xo1 : xe1) * c1, p21 = (up1 ? xe1 : xo1) * s1;
            y0 = up0 ? p10 + p20 : p10 - p20;
            y1 = up1 ? p11 + p21 : p11 - p21;
        }
    }

    // ---- store: the wavefront writes the 256-byte key -----------------------
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.block_keys + (n * a.Bcap + b) * Di);
    dst[lane] = pack_bf16x2(y0, y1);
}

hipError_t launch_wave(const QsaArgs &a, hipStream_t stream)
{
    const int64_t nb_max = (a.kbs - 1 + a.L) / a.kbs;
    const int64_t items = a.N * (nb_max + 1);           // < 2^31 (checked by the caller)
    const int64_t per_xcd = (items + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(qsa_prepare_wave_kernel, dim3((uint32_t)(per_xcd * kXcds)), dim3(64), 0,
                       stream, a, nb_max, (uint32_t)per_xcd, (uint32_t)items);
    return hipGetLastError();
}

template <int PPT>
hipError_t launch_ppt(const QsaArgs &a, hipStream_t stream)
{
    const int64_t nb_max = (a.kbs - 1 + a.L) / a.kbs;
    const int64_t grid = a.N * (nb_max + 1);
    const int64_t rows_per_chunk = kStageBytes / (2 * a.Di);    // >= 2 since Di <= 4096
    // LDS: the row stage, then m[Di], z[Di] and one float for the rms
    const size_t lds = kStageBytes + (2 * (size_t)a.Di + 4) * sizeof(float);
    hipLaunchKernelGGL((qsa_prepare_kernel<PPT>), dim3((uint32_t)grid), dim3(kThreads), lds,
                       stream, a, nb_max, rows_per_chunk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qsa_prepare(const QsaArgs &a, hipStream_t stream)
{
    if (a.Di == kWaveDi && a.kbs <= kWaveMaxRows)
        return launch_wave(a, stream);
    const int64_t pairs = a.Di / 2;
    if (pairs <= kThreads) return launch_ppt<1>(a, stream);
    if (pairs <= 2 * kThreads) return launch_ppt<2>(a, stream);
    if (pairs <= 4 * kThreads) return launch_ppt<4>(a, stream);
    return launch_ppt<8>(a, stream);
}

}  // namespace kvrc
