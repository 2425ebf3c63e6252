// Block selection over QSAPrepare block keys for gfx950 (MI355X): compressed
// attention scores, selection pooling, head-group sum and top-k.
//
// Computes, per sequence n (aclnnNsaCompressAttentionInfer, Formulas; the
// compressed keys are the block keys of openvino.opset17.qsa_prepare):
//   nb        = key_length[n] / kbs complete blocks
//   P_cmp[h]  = softmax_i(scale * q[n, h] . K[n, i]),  i < nb
//   Q[i]      = sum_h P_cmp[h][i]                      (all H heads share the key)
//   P[j]      = sum_{m < sel} sum_{c < cmp} Q[sel * j - m - c],  out-of-range terms 0,
//               for j < J = (nb + sel + cmp - 3) / sel + 1
//   indices   = the topk largest P[j], descending, equal scores by ascending j,
//               -1 where fewer than topk blocks exist
//
// Design (one 256-thread workgroup per sequence):
//   * the scores are a dense contraction (H x nb x Di), so they run on the
//     matrix cores (v_mfma_f32_16x16x32_bf16) from q [H, Di] staged in LDS;
//     wavefront w takes the 16-block tiles w, w + 4, ...;
//   * the sequence's keys pass through LDS in chunks of up to `chunk` rows,
//     each loaded by all threads at once (one memory latency per chunk);
//     every staged 16-row tile feeds all head tiles;
//   * the chunk's scores stay in LDS in log2 units (scale * log2 e * q . k),
//     so the softmax is a maximum, exp2 and a sum per head, and the head
//     sum Q[i] takes one reciprocal per head; a sequence that fits one chunk
//     takes one sweep of the matrix cores, a longer one three (maxima, sums,
//     Q), each recomputing the chunk's scores;
//   * pooling on LDS; the top-k on wavefront 0 alone: one arg-max of
//     (score, -index) per selected block, with no workgroup barrier.
// Float32 throughout (exp2f of the device library); deterministic: every
// reduction has a fixed order.
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// rows x pieces 16-byte pieces of a row-major bf16 matrix (row length Di) into
// LDS rows of rowb bytes; each thread issues kBatch loads before it stores
// any, so a batch costs one memory latency. Loads and stores are
// unconditional (indices past the end repeat the last piece) so that the
// batch stays in registers.
constexpr int kBatch = 8;

__device__ __forceinline__ const uint4 *piece_src(const uint16_t *src, int c, int pieces, int Di)
{
    return reinterpret_cast<const uint4 *>(src + (int64_t)(c / pieces) * Di + (c % pieces) * 8);
}

__device__ __forceinline__ uint4 *piece_dst(unsigned char *dst, int c, int pieces, int rowb)
{
    return reinterpret_cast<uint4 *>(dst + (c / pieces) * rowb + (c % pieces) * 16);
}

__device__ __forceinline__ void copy_rows(unsigned char *dst, const uint16_t *src, int rows,
                                          int pieces, int rowb, int Di, int tid)
{
    static_assert(kBatch == 8, "the batch below is spelled out for 8 pieces");
    const int total = rows * pieces;
    for (int c0 = tid; c0 < total; c0 += kThreads * kBatch) {
        // past the end: the last piece again (loads and stores stay unconditional,
        // so the batch lives in named registers)
        const int c1 = min(c0 + 1 * kThreads, total - 1), c2 = min(c0 + 2 * kThreads, total - 1);
        const int c3 = min(c0 + 3 * kThreads, total - 1), c4 = min(c0 + 4 * kThreads, total - 1);
        const int c5 = min(c0 + 5 * kThreads, total - 1), c6 = min(c0 + 6 * kThreads, total - 1);
        const int c7 = min(c0 + 7 * kThreads, total - 1);
        const uint4 v0 = *piece_src(src, c0, pieces, Di), v1 = *piece_src(src, c1, pieces, Di);
        const uint4 v2 = *piece_src(src, c2, pieces, Di), v3 = *piece_src(src, c3, pieces, Di);
        const uint4 v4 = *piece_src(src, c4, pieces, Di), v5 = *piece_src(src, c5, pieces, Di);
        const uint4 v6 = *piece_src(src, c6, pieces, Di), v7 = *piece_src(src, c7, pieces, Di);
        *piece_dst(dst, c0, pieces, rowb) = v0;
        *piece_dst(dst, c1, pieces, rowb) = v1;
        *piece_dst(dst, c2, pieces, rowb) = v2;
        *piece_dst(dst, c3, pieces, rowb) = v3;
        *piece_dst(dst, c4, pieces, rowb) = v4;
        *piece_dst(dst, c5, pieces, rowb) = v5;
        *piece_dst(dst, c6, pieces, rowb) = v6;
        *piece_dst(dst, c7, pieces, rowb) = v7;
    }
}

__global__ __launch_bounds__(kThreads) void qsa_select_kernel(QsaSelectArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = blockIdx.x;
    const int H = (int)a.H, Di = (int)a.Di;
    const int Jcap = (int)a.Jcap, KC = (int)a.chunk;

    // LDS: q [H][Di] and a key chunk [KC][Di] (bf16 rows padded by 16 bytes),
    // the chunk's scores S [H][KC + 4] (float32, log2 units), head max and
    // reciprocal sums [H] x 2, Q [Bcap], P [Jcap]
    const int rowb = Di * 2 + 16;
    const int srow = KC + 4;
    unsigned char *q_lds = smem;
    unsigned char *k_lds = smem + H * rowb;
    float *S = reinterpret_cast<float *>(k_lds + KC * rowb);
    float *hmax = S + H * srow;
    float *hrz = hmax + H;
    float *Q = hrz + H;                        // [Bcap]
    float *P = Q + a.Bcap;                     // [Jcap]

    const int64_t K = a.key_length[a.klc == 1 ? 0 : n];
    const int64_t nb64 = K >= 0 ? K / a.kbs : -1;
    float *scores = a.scores + n * Jcap;
    int32_t *out_idx = a.indices + n * a.topk;
    if (nb64 < 0 || nb64 > a.Bcap) {
        // invalid length: the sequence gets empty outputs and is counted
        for (int j = tid; j < Jcap; j += kThreads)
            scores[j] = 0.0f;
        for (int p = tid; p < a.topk; p += kThreads)
            out_idx[p] = -1;
        if (tid == 0 && a.err)
            atomicAdd(a.err, 1);
        return;
    }
    const int nb = (int)nb64;
    const int sel = (int)a.sel, cmpr = (int)a.cmp;
    const int J = nb == 0 ? 0 : (nb + sel + cmpr - 3) / sel + 1;
    const int pieces = Di / 8;                  // 16-byte pieces per row
    // scores in log2 units: softmax(x) = exp2(x log2(e) - max) / sum
    const float scale2 = a.scale * 1.44269504088896341f;

    copy_rows(q_lds, a.query + n * (int64_t)H * Di, H, pieces, rowb, Di, tid);
    for (int h = tid; h < H; h += kThreads) {
        hmax[h] = -INFINITY;
        hrz[h] = 0.0f;
    }
    for (int i = tid; i < a.Bcap; i += kThreads)
        Q[i] = 0.0f;

    const uint16_t *kn = a.keys + n * a.Bcap * (int64_t)Di;
    const int fr = lane & 15, fk = (lane >> 4) * 8;      // fragment row, first K element

    // keys [c0, c0 + rows) -> LDS, then S[h][i] = scale2 * q_h . k_(c0+i) for
    // i < rows (tiles of 16 x 16 on the matrix cores; wavefront w takes the
    // 16-row tiles w, w + 4, ...; the lanes of rows past `rows` are not stored)
    auto chunk_scores = [&](int c0, int rows) {
        __syncthreads();                                 // the previous chunk is used up
        copy_rows(k_lds, kn + (int64_t)c0 * Di, rows, pieces, rowb, Di, tid);
        __syncthreads();
        const int ntile = (rows + 15) / 16;
        for (int jt = wave; jt < ntile; jt += kWaves) {
            const unsigned char *kr = k_lds + (16 * jt + fr) * rowb + fk * 2;
            for (int ht = 0; ht < H / 16; ++ht) {
                const unsigned char *qa = q_lds + (16 * ht + fr) * rowb + fk * 2;
                // Di >= 32 (checked on the host): a do-while leaves no zero-trip
                // path, whose join with the MFMA path made the compiler read
                // the first accumulator register without the wait states an
                // MFMA result needs (it returned the stale initial value)
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                int k0 = 0;
                do {
                    const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(kr + k0 * 2);
                    const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(qa + k0 * 2);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, acc, 0, 0, 0);
                    k0 += 32;
                } while (k0 < Di);
                const int i = 16 * jt + fr;
                if (i < rows) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[(16 * ht + 4 * (lane >> 4) + r) * srow + i] = scale2 * acc[r];
                }
            }
        }
        __syncthreads();
    };
    // per head (wavefront w takes heads w, w + 4, ...; lanes stride the rows):
    // the running maximum over this chunk's rows
    auto chunk_max = [&](int rows) {
        for (int h = wave; h < H; h += kWaves) {
            float m = -INFINITY;
            for (int i = lane; i < rows; i += 64)
                m = fmaxf(m, S[h * srow + i]);
#pragma unroll
            for (int x = 32; x >= 1; x >>= 1)
                m = fmaxf(m, __shfl_xor(m, x, 64));
            if (lane == 0)
                hmax[h] = fmaxf(hmax[h], m);
        }
    };
    // per head: exp2(S - max) in place, its sum added to hrz (turned into
    // 1 / sum once every chunk is in)
    auto chunk_exp_sum = [&](int rows) {
        for (int h = wave; h < H; h += kWaves) {
            const float m = hmax[h];
            float z = 0.0f;
            for (int i = lane; i < rows; i += 64) {
                const float e = exp2f(S[h * srow + i] - m);
                S[h * srow + i] = e;
                z += e;
            }
#pragma unroll
            for (int x = 32; x >= 1; x >>= 1)
                z += __shfl_xor(z, x, 64);
            if (lane == 0)
                hrz[h] += z;
        }
    };
    // Q[c0 + i] = sum_h S[h][i] / sum_h with S holding exp2(s - max)
    auto chunk_q = [&](int c0, int rows) {
        for (int i = tid; i < rows; i += kThreads) {
            float q = 0.0f;
            for (int h = 0; h < H; ++h)
                q += S[h * srow + i] * hrz[h];
            Q[c0 + i] = q;
        }
    };
    auto finish_sums = [&]() {
        __syncthreads();
        for (int h = tid; h < H; h += kThreads)
            hrz[h] = 1.0f / hrz[h];
        __syncthreads();
    };

    if (nb > 0 && nb <= KC) {
        // the whole sequence in one chunk: one sweep of the matrix cores
        chunk_scores(0, nb);
        chunk_max(nb);
        __syncthreads();
        chunk_exp_sum(nb);
        finish_sums();
        chunk_q(0, nb);
    } else if (nb > KC) {
        for (int c0 = 0; c0 < nb; c0 += KC) {
            chunk_scores(c0, min(KC, nb - c0));
            chunk_max(min(KC, nb - c0));
        }
        for (int c0 = 0; c0 < nb; c0 += KC) {
            chunk_scores(c0, min(KC, nb - c0));
            chunk_exp_sum(min(KC, nb - c0));
        }
        finish_sums();
        for (int c0 = 0; c0 < nb; c0 += KC) {
            chunk_scores(c0, min(KC, nb - c0));
            for (int h = wave; h < H; h += kWaves) {
                const float m = hmax[h];
                for (int i = lane; i < min(KC, nb - c0); i += 64)
                    S[h * srow + i] = exp2f(S[h * srow + i] - m);
            }
            __syncthreads();
            chunk_q(c0, min(KC, nb - c0));
        }
    }
    __syncthreads();

    // ---- pooling ------------------------------------------------------------
    for (int j = tid; j < Jcap; j += kThreads) {
        float v = 0.0f;
        if (j < J) {
            for (int mm = 0; mm < sel; ++mm)
                for (int c = 0; c < cmpr; ++c) {
                    const int i = sel * j - mm - c;
                    if (i >= 0 && i < nb)
                        v += Q[i];
                }
        }
        scores[j] = v;
        P[j] = j < J ? v : -1.0f;                        // -1: not a candidate
    }
    __syncthreads();
    if (wave != 0)
        return;

    // ---- top-k on wavefront 0: repeated arg-max (score descending, index
    // ascending); a taken block is marked -1 ------------------------------------
    for (int p = 0; p < a.topk; ++p) {
        float bv = -1.0f;
        int bi = 0x7fffffff;
        for (int j = lane; j < J; j += 64) {
            const float v = P[j];
            if (v > bv || (v == bv && j < bi)) {
                bv = v;
                bi = j;
            }
        }
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) {
            const float v2 = __shfl_xor(bv, x, 64);
            const int i2 = __shfl_xor(bi, x, 64);
            if (v2 > bv || (v2 == bv && i2 < bi)) {
                bv = v2;
                bi = i2;
            }
        }
        const bool found = bv >= 0.0f && bi < J;       // every lane holds the winner
        if (lane == 0) {
            out_idx[p] = found ? bi : -1;
            if (found)
                P[bi] = -1.0f;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (!found) {
            for (int q = p + 1 + lane; q < a.topk; q += 64)
                out_idx[q] = -1;
            break;
        }
    }
}

}  // namespace

int64_t qsa_select_lds_bytes(int64_t H, int64_t Di, int64_t Bcap, int64_t Jcap, int64_t chunk)
{
    return (H + chunk) * (Di * 2 + 16) + 4 * (H * (chunk + 4) + 2 * H + Bcap + Jcap);
}

hipError_t launch_qsa_select(const QsaSelectArgs &a, hipStream_t stream)
{
    const int64_t lds = qsa_select_lds_bytes(a.H, a.Di, a.Bcap, a.Jcap, a.chunk);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qsa_select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(qsa_select_kernel, dim3((uint32_t)a.N), dim3(kThreads), (uint32_t)lds,
                       stream, a);
    return hipGetLastError();
}

}  // namespace kvrc
