// QSAPrepare block keys for gfx950 (openvino.opset17.qsa_prepare: one key
// per complete key block = mean of the block's key_block_size raw keys,
// RMS-normalised with k_norm_weight and rotated with the RoPE of the block's
// first token; only blocks completed by the new tokens are computed).
//
// Work decomposition: one wavefront per (sequence, new block), plus one
// wavefront per sequence that writes the carry state for the next call.
// The host cannot see key_length (it stays in device memory), so the grid is
// sized for the largest possible number of new blocks, floor((kbs-1+L)/kbs),
// and a wavefront whose block does not exist returns at once.
//
// Block mean: lane l owns dimension pairs l, l+64, ...; the kbs rows are read
// one row per load instruction (a fully coalesced Di*2-byte row), 16 rows in
// flight at a time, and each lane adds them in token order, so the float32
// sum has the same order as the definition whatever the chunking of the
// token stream across calls. The mean goes through LDS once so that the
// norm can use the canonical chunk layout of the square sum (8 dims per
// chunk, partials folded in halves), then the RoPE pairs are formed in LDS.
#include "device_common.hpp"
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

constexpr int kRowsInFlight = 16;

// Row of history token tau of sequence n (see qsa_prepare in kvrc.h).
__device__ __forceinline__ const uint16_t *history_row(const QsaArgs &a, int64_t n, int64_t tau,
                                                      int64_t P, int64_t r)
{
    if (tau < P)
        return a.past_raw + (n * (a.kbs - 1) + (tau - (P - r))) * a.Di;
    return a.raw + (n * a.L + (tau - P)) * a.Di;
}

template <int NP>   // dimension pairs per lane: Di/2 <= 64*NP
__global__ __launch_bounds__(64) void qsa_prepare_kernel(QsaArgs a, int64_t nb_max)
{
    extern __shared__ float lds[];        // m[Di], z[Di]
    const int lane = threadIdx.x;
    const int64_t per = nb_max + 1;
    const int64_t n = blockIdx.x / per;
    const int64_t j = blockIdx.x % per;
    const int64_t K = a.key_length[a.klc == 1 ? 0 : n];
    const int64_t kbs = a.kbs, Di = a.Di, L = a.L;
    if (K < L || K / kbs > a.Bcap) {
        if (j == 0 && lane == 0 && a.err)
            atomicAdd(a.err, 1);
        return;
    }
    const int64_t P = K - L;
    const int64_t r = P % kbs;

    if (j == nb_max) {
        // ---- carry state: tokens [t1, K) of the incomplete block ----------
        const int64_t r2 = K % kbs, t1 = K - r2;
        const int64_t nvec = Di / 8;
        for (int64_t e = lane; e < r2 * nvec; e += 64) {
            const int64_t i = e / nvec, c = e % nvec;
            const uint16_t *src = history_row(a, n, t1 + i, P, r) + 8 * c;
            *reinterpret_cast<uint4 *>(a.next_raw + (n * (kbs - 1) + i) * Di + 8 * c) =
                *reinterpret_cast<const uint4 *>(src);
        }
        if (a.rope_cos && r2 > 0) {
            const int64_t Dr = a.Dr;
            for (int64_t d = lane; d < Dr; d += 64) {
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

    // ---- block mean: float32 sum in token order --------------------------
    const int64_t npairs = Di / 2;
    float acc[2 * NP];
#pragma unroll
    for (int k = 0; k < 2 * NP; ++k)
        acc[k] = 0.0f;
    const int64_t tau0 = b * kbs;
    for (int64_t base = 0; base < kbs; base += kRowsInFlight) {
        const int64_t cnt = kbs - base < kRowsInFlight ? kbs - base : kRowsInFlight;
        uint32_t w[kRowsInFlight][NP];
#pragma unroll
        for (int q = 0; q < kRowsInFlight; ++q) {
            if (q < cnt) {
                const uint16_t *row = history_row(a, n, tau0 + base + q, P, r);
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    const int64_t p = lane + 64 * k;
                    w[q][k] = p < npairs ? *reinterpret_cast<const uint32_t *>(row + 2 * p) : 0u;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kRowsInFlight; ++q) {
            if (q < cnt) {
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    acc[2 * k] = acc[2 * k] + bf16_lo(w[q][k]);
                    acc[2 * k + 1] = acc[2 * k + 1] + bf16_hi(w[q][k]);
                }
            }
        }
    }
    float *m = lds;
    float *z = lds + Di;
    const float fk = (float)kbs;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int64_t p = lane + 64 * k;
        if (p < npairs) {
            m[2 * p] = acc[2 * k] / fk;
            m[2 * p + 1] = acc[2 * k + 1] / fk;
        }
    }
    __syncthreads();

    // ---- RMS normalisation over Di (canonical square sum) ----------------
    const int64_t nch = Di / 8;
    if (a.weight) {
        float part = 0.0f;
        for (int64_t c = lane; c < nch; c += 64) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = m[8 * c + e];
            part = chunk_sumsq(x, part);
        }
        const float ss = fold_sum<64>(part);
        const float ms = ss / (float)Di;
        const float rms = sqrtf(ms + a.eps);
        for (int64_t d = lane; d < Di; d += 64) {
            const float q = m[d] / rms;
            z[d] = q * __uint_as_float((uint32_t)a.weight[d] << 16);
        }
    } else {
        for (int64_t d = lane; d < Di; d += 64)
            z[d] = m[d];
    }
    __syncthreads();

    // ---- RoPE of the trailing Dr dims with the first token's cos/sin -----
    // The rotated values go to the (no longer needed) mean buffer m[0, Dr).
    const int64_t Dr = a.rope_cos ? a.Dr : 0;
    const int64_t base = Di - Dr;
    if (Dr) {
        const int64_t h = Dr / 2;
        const float *cr, *sr;
        if (tau0 < P) {
            cr = a.past_rope + n * 2 * Dr;
            sr = cr + Dr;
        } else {
            cr = a.rope_cos + (n * L + (tau0 - P)) * Dr;
            sr = a.rope_sin + (n * L + (tau0 - P)) * Dr;
        }
        for (int64_t o = lane; o < Dr; o += 64) {
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
    for (int64_t c = lane; c < nch; c += 64) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t d = 8 * c + e;
            v[e] = d < base ? z[d] : m[d - base];
        }
        *reinterpret_cast<uint4 *>(dst + 8 * c) = pack8(v);
    }
}

template <int NP>
hipError_t launch_np(const QsaArgs &a, hipStream_t stream)
{
    const int64_t nb_max = (a.kbs - 1 + a.L) / a.kbs;
    const int64_t grid = a.N * (nb_max + 1);
    const size_t lds = 2 * (size_t)a.Di * sizeof(float);
    hipLaunchKernelGGL((qsa_prepare_kernel<NP>), dim3((uint32_t)grid), dim3(64), lds, stream, a,
                       nb_max);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qsa_prepare(const QsaArgs &a, hipStream_t stream)
{
    const int64_t pairs = a.Di / 2;
    if (pairs <= 64) return launch_np<1>(a, stream);
    if (pairs <= 128) return launch_np<2>(a, stream);
    if (pairs <= 256) return launch_np<4>(a, stream);
    if (pairs <= 512) return launch_np<8>(a, stream);
    if (pairs <= 1024) return launch_np<16>(a, stream);
    return launch_np<32>(a, stream);
}

}  // namespace kvrc
