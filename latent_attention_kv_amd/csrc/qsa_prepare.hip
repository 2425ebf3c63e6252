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
    const int64_t pairs = a.Di / 2;
    if (pairs <= kThreads) return launch_ppt<1>(a, stream);
    if (pairs <= 2 * kThreads) return launch_ppt<2>(a, stream);
    if (pairs <= 4 * kThreads) return launch_ppt<4>(a, stream);
    return launch_ppt<8>(a, stream);
}

}  // namespace kvrc
