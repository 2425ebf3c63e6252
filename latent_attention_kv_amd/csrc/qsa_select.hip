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
// Design (one 512-thread workgroup per sequence, both kernels):
//   * the scores are a dense contraction (H x nb x Di), so they run on the
//     matrix cores (v_mfma_f32_16x16x32_bf16); wavefront w takes the
//     16-block column tiles w, w + 8, ... and every head tile of each;
//   * scores in log2 units (scale * log2 e * q . k): the softmax is a
//     maximum, exp2 and a sum per head, and Q takes one reciprocal per head;
//   * qsa_select_fast_kernel (Di / 32, H / 16 and the column tiles per
//     wavefront known at compile time): keys as the A operand, so each lane
//     holds one head of 4 blocks per tile and a head's statistics stay in
//     the lane; key fragments go straight into registers, requested with q
//     and the key length when the workgroup starts; the per-lane softmax
//     partials meet once in LDS (maximum, sum and a factor per partial);
//   * qsa_select_kernel (every other shape): q as the A operand, a tile's
//     accumulator holds 4 heads x 16 blocks per 16-lane row, so a head's
//     maximum or sum over a tile is four DPP steps inside the row, partial
//     results combined per head in a fixed order; keys staged in LDS chunks; a
//     sequence that fits one chunk with few enough tiles per wavefront keeps
//     its scores in registers, a longer one takes three sweeps over its
//     chunks (maxima, sums, Q), each recomputing its tiles;
//   * pooling on LDS; top-k by rank: every block gets a 64-bit key (score
//     above, index below) and lands at the number of larger keys, counted by
//     four lanes per candidate (up to 128 candidates) or in segments spread
//     over the workgroup; above kRankMax candidates, repeated arg-max on one
//     wavefront.
// Float32 throughout (exp2f of the device library); deterministic: every
// floating-point reduction has a fixed order.
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRankMax = 2048;
constexpr int kMaxTiles = 16;            // score tiles a wavefront holds in registers
constexpr int kPartStride = 4 * kWaves + 1; // fast kernel: lane partials per head (+1: banks)

// rows_a rows of a, then rows of b (row-major bf16, row length Di, 16-byte
// pieces) into consecutive LDS rows of rowb bytes. Each thread issues kBatch
// loads before it stores any, so a batch costs one memory latency. Indices
// past the end repeat the last piece (load and store), so every load and
// store is unconditional: a conditional store lets the compiler move its load
// into the branch, after the wait for the previous one.
constexpr int kBatch = 12;

struct RowSrc {
    const uint16_t *a, *b;
    int rows_a, pieces, Di;
    __device__ __forceinline__ const uint4 *at(int c) const
    {
        const int row = c / pieces, off = (c % pieces) * 8;
        const uint16_t *p = row < rows_a ? a + (int64_t)row * Di : b + (int64_t)(row - rows_a) * Di;
        return reinterpret_cast<const uint4 *>(p + off);
    }
};

// one piece of the batch: load (index past the end -> the last piece) and store
#define KVRC_SEL_LOAD(i) const uint4 v##i = *src.at(min(c0 + (i) * kThreads, total - 1));
#define KVRC_SEL_STORE(i)                                                                    \
    {                                                                                        \
        const int c = min(c0 + (i) * kThreads, total - 1);                                   \
        *reinterpret_cast<uint4 *>(dst + (c / pieces) * rowb + (c % pieces) * 16) = v##i;    \
    }

__device__ __forceinline__ void copy_rows(unsigned char *dst, const RowSrc &src, int rows, int rowb,
                                          int tid)
{
    static_assert(kBatch == 12, "the batch below is spelled out for 12 pieces");
    const int pieces = src.pieces;
    const int total = rows * pieces;
    for (int c0 = tid; c0 < total; c0 += kThreads * kBatch) {
        KVRC_SEL_LOAD(0) KVRC_SEL_LOAD(1) KVRC_SEL_LOAD(2) KVRC_SEL_LOAD(3)
        KVRC_SEL_LOAD(4) KVRC_SEL_LOAD(5) KVRC_SEL_LOAD(6) KVRC_SEL_LOAD(7)
        KVRC_SEL_LOAD(8) KVRC_SEL_LOAD(9) KVRC_SEL_LOAD(10) KVRC_SEL_LOAD(11)
        __builtin_amdgcn_sched_barrier(0);               // every load issued before the first wait
        KVRC_SEL_STORE(0) KVRC_SEL_STORE(1) KVRC_SEL_STORE(2) KVRC_SEL_STORE(3)
        KVRC_SEL_STORE(4) KVRC_SEL_STORE(5) KVRC_SEL_STORE(6) KVRC_SEL_STORE(7)
        KVRC_SEL_STORE(8) KVRC_SEL_STORE(9) KVRC_SEL_STORE(10) KVRC_SEL_STORE(11)
    }
}
#undef KVRC_SEL_LOAD
#undef KVRC_SEL_STORE

// DPP inside a 16-lane row: xor 1, xor 2 (quad permutes), then the half-row
// and row mirrors; after the four steps every lane of the row holds the
// reduction of all 16 (the same value in every lane: each step combines two
// equal partial results, and + and max are commutative)
template <int kCtrl>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRor8 = 0x128;         // row_ror:8 (in a 16-lane row: lane xor 8)

// Workgroup barrier that orders LDS only: its fences wait for this thread's
// LDS operations, not for its global loads and stores (__syncthreads waits for
// both). For barriers between LDS producers and consumers where no thread
// reads global memory another thread of the workgroup wrote.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The maximum steps are single v_max_f32_dpp instructions. The values are
// results of arithmetic (never signalling NaNs), so the IEEE-mode v_max_f32
// already returns what fmaxf would (a quiet NaN operand yields the other
// one); written with fmaxf, each step also quiets its DPP operand and loads
// an unused "old" value, three instructions more. Each step starts with the
// two wait states a DPP read needs after the VALU write of its source.
__device__ __forceinline__ float row_max16(float v)
{
    float r;
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(v));
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                 : "=v"(v) : "v"(r));
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(v));
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf"
                 : "=v"(v) : "v"(r));
    return v;
}

__device__ __forceinline__ float row_sum16(float v)
{
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v + dpp<kDppMirror>(v);
}

// one 16 x 16 tile: rows = heads (fragment of q at qa), columns = blocks
// (fragment of the staged keys at kr). Di >= 32 (checked on the host): a
// do-while leaves no path on which no MFMA runs, whose join with the MFMA path
// made the compiler read the first accumulator register without the wait
// states an MFMA result needs.
__device__ __forceinline__ f32x4 score_tile(const unsigned char *qa, const unsigned char *kr, int Di)
{
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    int k0 = 0;
    do {
        const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(kr + k0 * 2);
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(qa + k0 * 2);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, acc, 0, 0, 0);
        k0 += 32;
    } while (k0 < Di);
    return acc;
}

// The sequence's block count nb = key_length / kbs, or -1 for an invalid
// length (negative, or more blocks than the capacity): such a sequence gets
// scores 0 and indices -1 here and counts once in the error counter.
__device__ __forceinline__ int sequence_blocks_of(const QsaSelectArgs &a, int64_t K, float *scores,
                                                  int32_t *out_idx, int tid)
{
    const int64_t nb = K >= 0 ? K / a.kbs : -1;
    if (nb >= 0 && nb <= a.Bcap)
        return (int)nb;
    for (int j = tid; j < a.Jcap; j += kThreads)
        scores[j] = 0.0f;
    for (int p = tid; p < a.topk; p += kThreads)
        out_idx[p] = -1;
    if (tid == 0 && a.err)
        atomicAdd(a.err, 1);
    return -1;
}

__device__ __forceinline__ int sequence_blocks(const QsaSelectArgs &a, int64_t n, float *scores,
                                               int32_t *out_idx, int tid)
{
    return sequence_blocks_of(a, a.key_length[a.klc == 1 ? 0 : n], scores, out_idx, tid);
}

// Pooling of Q [nb] into the J selection-block scores, and the top-k. Q is
// complete in LDS (the caller's barrier). LDS scratch: P [Jcap rounded up to
// 4] (float scores), and for the rank top-k K [up to kRankMax] (64-bit keys)
// and R [up to kRankMax] (ranks).
__device__ __forceinline__ void pool_and_select(const QsaSelectArgs &a, const float *Q, float *P,
                                                uint64_t *K, int *R, int nb, int J, float *scores,
                                                int32_t *out_idx, int tid, int lane, int wave)
{
    const int sel = (int)a.sel, cmpr = (int)a.cmp, Jcap = (int)a.Jcap;
    const int Jcap4 = (Jcap + 3) / 4 * 4, J4 = (J + 3) / 4 * 4;
    const bool by_rank = J <= kRankMax;
    for (int j = tid; j < Jcap4; j += kThreads) {
        float v = 0.0f;
        if (j < J) {
            for (int mm = 0; mm < sel; ++mm)
                for (int c = 0; c < cmpr; ++c) {
                    const int i = sel * j - mm - c;
                    if (i >= 0 && i < nb)
                        v += Q[i];
                }
        }
        if (j < Jcap)
            scores[j] = v;
        // -1 marks what is never selected: blocks past J and NaN scores
        P[j] = j < J && v == v ? v : -1.0f;
        if (by_rank && j < J4) {
            // one 64-bit key orders the blocks: score (its bits + 1; scores
            // are >= +0) above, 2^32 - 1 - j below (equal scores: the lower
            // index first); NaN scores and the padding past J get 0 / lower
            // halves only, below every real score
            const uint32_t hi = j < J && v == v ? (v > 0.0f ? __float_as_uint(v) : 0u) + 1u : 0u;
            K[j] = j < J ? ((uint64_t)hi << 32) | (0xFFFFFFFFu - (uint32_t)j) : 0ull;
            R[j] = 0;
        }
    }
    lds_barrier();

    if (J <= kThreads / 4) {
        // ---- top-k by rank, up to 128 blocks: the position of block j is
        // the number of keys above its own (ranks 0 .. J-1, each once),
        // counted by the four lanes 4 j .. 4 j + 3, lane r over the key pairs
        // 4 t + r (the four lanes of a quad read 64 consecutive bytes), and
        // added over the quad in two DPP steps
        // (every read is issued before the first compare: pairs past the
        // keys reread the last pair and count nothing)
        const int j = tid >> 2, r = tid & 3;
        const uint64_t key = j < J ? K[j] : 0ull;
        int cnt = 0;
        if (j < J) {
            constexpr int kPairs = kThreads / 4 / 2 / 4;  // pairs per lane at 128 keys
            ulonglong2 kk[kPairs];
#pragma unroll
            for (int t = 0; t < kPairs; ++t)
                kk[t] = *reinterpret_cast<const ulonglong2 *>(K + 2 * min(r + 4 * t, J4 / 2 - 1));
#pragma unroll
            for (int t = 0; t < kPairs; ++t) {
                const bool in = 2 * (r + 4 * t) < J4;
                cnt += in && kk[t].x > key;
                cnt += in && kk[t].y > key;
            }
        }
        cnt += __builtin_amdgcn_update_dpp(0, cnt, kDppXor1, 0xF, 0xF, false);
        cnt += __builtin_amdgcn_update_dpp(0, cnt, kDppXor2, 0xF, 0xF, false);
        if (j < J && r == 0 && cnt < a.topk)
            out_idx[cnt] = (key >> 32) != 0 ? j : -1;        // a NaN score leaves -1
        for (int p = J + tid; p < a.topk; p += kThreads)
            out_idx[p] = -1;
        return;
    }
    if (by_rank) {
        // ---- top-k by rank: the position of block j is the number of keys
        // above its own (ranks 0 .. J-1, each once). The count for each block
        // is split into S segments of the key list, so that the work spreads
        // over the workgroup; the partial counts are added in LDS (integer,
        // so the order does not matter).
        const int S = max(1, min(kThreads / max(J, 1), 16));
        const int L = ((J4 + S - 1) / S + 1) & ~1;      // keys per segment, even
        for (int w = tid; w < J * S; w += kThreads) {
            const int seg = w / J, j = w - seg * J;      // neighbouring lanes: same segment
            const uint64_t key = K[j];
            const int lo = seg * L, hi = min(lo + L, J4);
            int cnt = 0;
#pragma unroll 4
            for (int jj = lo; jj < hi; jj += 2) {
                const ulonglong2 kk = *reinterpret_cast<const ulonglong2 *>(K + jj);
                cnt += kk.x > key;
                cnt += kk.y > key;
            }
            atomicAdd(R + j, cnt);
        }
        lds_barrier();
        for (int j = tid; j < J; j += kThreads) {
            const int rank = R[j];
            if (rank < a.topk)
                out_idx[rank] = (K[j] >> 32) != 0 ? j : -1;   // a NaN score leaves -1
        }
        for (int p = J + tid; p < a.topk; p += kThreads)
            out_idx[p] = -1;
        return;
    }
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

__global__ __launch_bounds__(kThreads) void qsa_select_kernel(QsaSelectArgs a)
{
    // no contraction: scale2 * acc - max is rounded alike wherever it is
    // computed
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = blockIdx.x;
    const int H = (int)a.H, Di = (int)a.Di;
    const int Jcap = (int)a.Jcap, KC = (int)a.chunk;

    // LDS: q [H][Di] and a key chunk [KC][Di] (bf16 rows padded by 16 bytes),
    // per-wavefront head maxima and sums [kWaves][H] x 2, the combined head
    // maxima and reciprocal sums [H] x 2, per-tile head maxima and sums
    // [KC / 16][H] x 2, Q [Bcap], P [Jcap] (both rounded up to 4), the rank
    // keys and ranks [min(Jcap rounded up to 4, kRankMax)] (8 + 4 bytes)
    const int rowb = Di * 2 + 16;
    unsigned char *q_lds = smem;
    unsigned char *k_lds = smem + H * rowb;
    float *wmax = reinterpret_cast<float *>(k_lds + KC * rowb);
    float *wsum = wmax + kWaves * H;
    float *hmax = wsum + kWaves * H;
    float *hrz = hmax + H;
    float *tmax = hrz + H;
    float *tsum = tmax + (KC / 16) * H;
    float *Q = tsum + (KC / 16) * H;
    float *P = Q + (a.Bcap + 3) / 4 * 4;
    uint64_t *K = reinterpret_cast<uint64_t *>(P + (Jcap + 3) / 4 * 4);
    int *R = reinterpret_cast<int *>(K + min((Jcap + 3) / 4 * 4, kRankMax));

    float *scores = a.scores + n * Jcap;
    int32_t *out_idx = a.indices + n * a.topk;
    const int nb = sequence_blocks(a, n, scores, out_idx, tid);
    if (nb < 0)
        return;
    const int sel = (int)a.sel, cmpr = (int)a.cmp;
    const int J = nb == 0 ? 0 : (nb + sel + cmpr - 3) / sel + 1;
    const int pieces = Di / 8;                  // 16-byte pieces per row
    const int HT = H / 16;
    // scores in log2 units: softmax(x) = exp2(x log2(e) - max) / sum
    const float scale2 = a.scale * 1.44269504088896341f;

    const uint16_t *qn = a.query + n * (int64_t)H * Di;
    const uint16_t *kn = a.keys + n * a.Bcap * (int64_t)Di;
    const int fr = lane & 15, g = lane >> 4;             // fragment row / column, lane group
    const int fk = g * 8;                                // first K element of the fragment
    const int ntile = (nb + 15) / 16;                    // column tiles of the sequence
    const bool in_regs = nb > 0 && nb <= KC && HT * ((ntile + kWaves - 1) / kWaves) <= kMaxTiles;

    if (in_regs) {
        copy_rows(q_lds, RowSrc{qn, kn, H, pieces, Di}, H + nb, rowb, tid);
        __syncthreads();
        // this wavefront's tiles: t -> (column tile jt, head tile ht), ht fastest
        const int T = wave < ntile ? ((ntile - 1 - wave) / kWaves + 1) * HT : 0;
        f32x4 e[kMaxTiles];
        {
            int ht = 0, jt = wave;
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                if (t < T) {
                    const f32x4 acc = score_tile(q_lds + (16 * ht + fr) * rowb + fk * 2,
                                                 k_lds + (16 * jt + fr) * rowb + fk * 2, Di);
                    const bool ok = 16 * jt + fr < nb;
                    f32x4 mx;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        e[t][q] = scale2 * acc[q];
                        mx[q] = row_max16(ok ? e[t][q] : -INFINITY);
                    }
                    if (fr == 0)
                        *reinterpret_cast<f32x4 *>(tmax + jt * H + 16 * ht + 4 * g) = mx;
                    if (++ht == HT) {
                        ht = 0;
                        jt += kWaves;
                    }
                }
            }
        }
        __syncthreads();
        for (int h = tid; h < H; h += kThreads) {
            float v = -INFINITY;
            for (int jt = 0; jt < ntile; ++jt)
                v = fmaxf(v, tmax[jt * H + h]);
            hmax[h] = v;
        }
        __syncthreads();
        {
            int ht = 0, jt = wave;
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                if (t < T) {
                    const bool ok = 16 * jt + fr < nb;
                    const f32x4 m = *reinterpret_cast<const f32x4 *>(hmax + 16 * ht + 4 * g);
                    f32x4 zs;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        e[t][q] = ok ? exp2f(e[t][q] - m[q]) : 0.0f;
                        zs[q] = row_sum16(e[t][q]);
                    }
                    if (fr == 0)
                        *reinterpret_cast<f32x4 *>(tsum + jt * H + 16 * ht + 4 * g) = zs;
                    if (++ht == HT) {
                        ht = 0;
                        jt += kWaves;
                    }
                }
            }
        }
        __syncthreads();
        for (int h = tid; h < H; h += kThreads) {
            float v = 0.0f;
            for (int jt = 0; jt < ntile; ++jt)
                v += tsum[jt * H + h];
            hrz[h] = 1.0f / v;
        }
        __syncthreads();
        {
            int ht = 0, jt = wave;
            float qv = 0.0f;
#pragma unroll
            for (int t = 0; t < kMaxTiles; ++t) {
                if (t < T) {
                    const f32x4 rz = *reinterpret_cast<const f32x4 *>(hrz + 16 * ht + 4 * g);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        qv += e[t][q] * rz[q];
                    if (++ht == HT) {
                        // the 4 lane groups hold the same block for different heads
                        qv += __shfl_xor(qv, 16, 64);
                        qv += __shfl_xor(qv, 32, 64);
                        if (g == 0 && 16 * jt + fr < nb)
                            Q[16 * jt + fr] = qv;
                        qv = 0.0f;
                        ht = 0;
                        jt += kWaves;
                    }
                }
            }
        }
    } else if (nb > 0) {
        for (int i = tid; i < kWaves * H; i += kThreads) {
            wmax[i] = -INFINITY;
            wsum[i] = 0.0f;
        }
        const int nchunk = (nb + KC - 1) / KC;
        // sweep 0: head maxima; sweep 1: head sums of exp2(s - max); sweep 2: Q
        for (int sweep = 0; sweep < 3; ++sweep) {
            for (int c = 0; c < nchunk; ++c) {
                const int c0 = c * KC, rows = min(KC, nb - c0);
                __syncthreads();                         // the previous chunk is used up
                if (sweep == 0 && c == 0)
                    copy_rows(q_lds, RowSrc{qn, kn, H, pieces, Di}, H + rows, rowb, tid);
                else
                    copy_rows(k_lds, RowSrc{kn + (int64_t)c0 * Di, nullptr, rows, pieces, Di},
                              rows, rowb, tid);
                __syncthreads();
                const int ctile = (rows + 15) / 16;
                if (wave >= ctile)
                    continue;
                if (sweep < 2) {
                    for (int ht = 0; ht < HT; ++ht) {
                        const unsigned char *qa = q_lds + (16 * ht + fr) * rowb + fk * 2;
                        const int h0 = 16 * ht + 4 * g;  // this lane's 4 heads
                        const f32x4 m = *reinterpret_cast<const f32x4 *>(hmax + h0);
                        f32x4 r = sweep == 0 ? f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY}
                                             : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        for (int jt = wave; jt < ctile; jt += kWaves) {
                            const f32x4 acc = score_tile(qa, k_lds + (16 * jt + fr) * rowb + fk * 2, Di);
                            const bool ok = 16 * jt + fr < rows;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float s = scale2 * acc[q];
                                if (sweep == 0)
                                    r[q] = ok ? fmaxf(r[q], s) : r[q];
                                else
                                    r[q] += ok ? exp2f(s - m[q]) : 0.0f;
                            }
                        }
                        float *dst = (sweep == 0 ? wmax : wsum) + wave * H + h0;
                        f32x4 old = *reinterpret_cast<const f32x4 *>(dst);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            old[q] = sweep == 0 ? fmaxf(old[q], row_max16(r[q])) : old[q] + row_sum16(r[q]);
                        if (fr == 0)
                            *reinterpret_cast<f32x4 *>(dst) = old;
                    }
                } else {
                    for (int jt = wave; jt < ctile; jt += kWaves) {
                        const unsigned char *kr = k_lds + (16 * jt + fr) * rowb + fk * 2;
                        float qv = 0.0f;
                        for (int ht = 0; ht < HT; ++ht) {
                            const int h0 = 16 * ht + 4 * g;
                            const f32x4 acc = score_tile(q_lds + (16 * ht + fr) * rowb + fk * 2, kr, Di);
                            const f32x4 m = *reinterpret_cast<const f32x4 *>(hmax + h0);
                            const f32x4 rz = *reinterpret_cast<const f32x4 *>(hrz + h0);
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                qv += exp2f(scale2 * acc[q] - m[q]) * rz[q];
                        }
                        qv += __shfl_xor(qv, 16, 64);
                        qv += __shfl_xor(qv, 32, 64);
                        const int i = 16 * jt + fr;
                        if (g == 0 && i < rows)
                            Q[c0 + i] = qv;
                    }
                }
            }
            __syncthreads();
            if (sweep < 2) {
                // combine the wavefronts in a fixed order; the next sweep's
                // first staging barrier orders it before any use
                for (int h = tid; h < H; h += kThreads) {
                    float v = sweep == 0 ? -INFINITY : 0.0f;
                    for (int w = 0; w < kWaves; ++w)
                        v = sweep == 0 ? fmaxf(v, wmax[w * H + h]) : v + wsum[w * H + h];
                    if (sweep == 0)
                        hmax[h] = v;
                    else
                        hrz[h] = 1.0f / v;
                }
            }
        }
    }
    __syncthreads();
    pool_and_select(a, Q, P, K, R, nb, J, scores, out_idx, tid, lane, wave);
}

// Fast path for the common shapes, all sizes known at compile time: Di = 32 DK,
// H = 16 HT, and at most JWM column tiles per wavefront (Bcap <= 128 JWM).
//
// The keys are the A operand (rows = blocks) and q the B operand (columns =
// heads), so lane (g, fr) of a tile holds head 16 ht + fr for blocks 4 g .. 4 g
// + 3 of it: a head's maximum and sum over the lane's blocks stay in the lane.
// Wavefront w takes column tiles w + 8 jl; each lane loads the key fragments
// of its tile rows straight into registers: those of the first tile when the
// workgroup starts, together with q and the key length (rows clamped to the
// capacity; a fragment past the sequence is loaded and never used), the
// others once the key length shows that their tile holds blocks of the
// sequence. q passes through LDS once; tiles past the sequence are skipped.
//
// Softmax per head over its 32 lane partials (8 wavefronts x 4 lane groups),
// in log2 units s = scale log2(e) q . k: lane partial p holds m_p = max s
// over its blocks and z_p = sum exp2(s - m_p); with M = max_p m_p and
// Z = sum_p z_p exp2(m_p - M), each score's softmax term is
// exp2(s - m_p) c_p with c_p = exp2(m_p - M) / Z, the factorisation of
// exp2(s - M) / Z over the partials (one pass over the scores, one exchange
// of partials through LDS). Q's head sum takes each lane's products over its
// head tiles, then the 16 head lanes of a tile row in four DPP steps.
template <int DK, int HT, int JWM>
__global__ __launch_bounds__(kThreads) void qsa_select_fast_kernel(QsaSelectArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int Di = 32 * DK, H = 16 * HT, rowb = 2 * Di + 16, pieces = Di / 8;
    constexpr int QP = H * pieces, QPT = (QP + kThreads - 1) / kThreads;
    // head tiles whose q fragments are held at once (at most 16 fragments =
    // 64 registers); with all of them held, q is read from LDS once
    constexpr int QF = 16 / DK < HT ? 16 / DK : HT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;             // fragment row / column, lane group
    const int64_t n = blockIdx.x;

    // LDS: q [H][Di] (rows padded by 16 bytes); per head its lane partials
    // m_p (then c_p) and z_p [H][kPartStride] x 2; Q [Bcap rounded up to 16];
    // P [Jcap], the rank keys and ranks as in pool_and_select
    const int rows16 = (int)(a.Bcap + 15) / 16 * 16;
    unsigned char *q_lds = smem;
    float *pm = reinterpret_cast<float *>(smem + H * rowb);
    float *pz = pm + H * kPartStride;
    float *Q = pz + H * kPartStride;
    float *P = Q + rows16;
    uint64_t *K = reinterpret_cast<uint64_t *>(P + (a.Jcap + 3) / 4 * 4);
    int *R = reinterpret_cast<int *>(K + min((int)(a.Jcap + 3) / 4 * 4, kRankMax));

    float *scores = a.scores + n * a.Jcap;
    int32_t *out_idx = a.indices + n * a.topk;
    const uint16_t *kn = a.keys + n * a.Bcap * (int64_t)Di;
    const int last = (int)a.Bcap - 1;
    auto load_keys = [&](bf16x8 *f, int jl) __attribute__((always_inline)) {
        const int row = min(16 * (wave + kWaves * jl) + fr, last);
#pragma unroll
        for (int u = 0; u < DK; ++u)
            f[u] = *reinterpret_cast<const bf16x8 *>(kn + (int64_t)row * Di + 32 * u + 8 * g);
    };
    // the key length, the q rows and the first tile's key fragments are all
    // requested before any of them is waited for
    const int64_t Klen = __builtin_nontemporal_load(a.key_length + (a.klc == 1 ? 0 : n));
    bf16x8 kf[JWM][DK];
    {
        const uint16_t *qn = a.query + n * (int64_t)H * Di;
        // (a vector type, not uint4: the struct copies of uint4 kept the
        // array in scratch memory here)
        u32x4 qs[QPT];
#pragma unroll
        for (int b = 0; b < QPT; ++b) {
            const int c = min(tid + b * kThreads, QP - 1);
            qs[b] = *reinterpret_cast<const u32x4 *>(qn + (c / pieces) * Di + (c % pieces) * 8);
        }
        load_keys(kf[0], 0);
#pragma unroll
        for (int b = 0; b < QPT; ++b) {
            const int c = min(tid + b * kThreads, QP - 1);
            *reinterpret_cast<u32x4 *>(q_lds + (c / pieces) * rowb + (c % pieces) * 16) = qs[b];
        }
    }
    const int nb = sequence_blocks_of(a, Klen, scores, out_idx, tid);
    if (nb < 0)
        return;
    const int sel = (int)a.sel, cmpr = (int)a.cmp;
    const int J = nb == 0 ? 0 : (nb + sel + cmpr - 3) / sel + 1;

    if (nb > 0) {
#pragma unroll
        for (int jl = 1; jl < JWM; ++jl)
            if (16 * (wave + kWaves * jl) < nb)
                load_keys(kf[jl], jl);
        const float scale2 = a.scale * 1.44269504088896341f;
        lds_barrier();                                   // q in LDS (the keys may still arrive)

        // scores (log2 units): e[jl][ht] = tile of column tile wave + 8 jl and
        // head tile ht, for the tiles that hold blocks of the sequence (each
        // MFMA result is read by the multiply in the same branch)
        f32x4 e[JWM][HT];
        bf16x8 qf[QF][DK];
        auto load_q = [&](int ht0) __attribute__((always_inline)) {
#pragma unroll
            for (int hq = 0; hq < QF; ++hq)
#pragma unroll
                for (int u = 0; u < DK; ++u)
                    qf[hq][u] = *reinterpret_cast<const bf16x8 *>(
                        q_lds + (16 * (ht0 + hq) + fr) * rowb + (32 * u + 8 * g) * 2);
            // every fragment is read before the first MFMA that needs one
#pragma unroll
            for (int hq = 0; hq < QF; ++hq)
#pragma unroll
                for (int u = 0; u < DK; ++u)
                    asm volatile("" ::"v"(qf[hq][u]));
        };
        if constexpr (QF == HT)
            load_q(0);
#pragma unroll
        for (int jl = 0; jl < JWM; ++jl) {
            if (16 * (wave + kWaves * jl) < nb) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    if constexpr (QF < HT)
                        if (ht % QF == 0)
                            load_q(ht);
                    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int u = 0; u < DK; ++u)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[jl][u], qf[ht % QF][u], acc,
                                                                      0, 0, 0);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        e[jl][ht][q] = scale2 * acc[q];
                }
            }
        }

        // this lane's maximum and minimum per head over its blocks of the
        // sequence (the tile the sequence ends in is masked)
        float hi[HT], lo[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            hi[ht] = -INFINITY;
            lo[ht] = INFINITY;
        }
#pragma unroll
        for (int jl = 0; jl < JWM; ++jl) {
            const int t0 = 16 * (wave + kWaves * jl);
            if (t0 + 16 <= nb) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    const f32x4 v = e[jl][ht];
                    hi[ht] = fmaxf(fmaxf(fmaxf(fmaxf(hi[ht], v[0]), v[1]), v[2]), v[3]);
                    lo[ht] = fminf(fminf(fminf(fminf(lo[ht], v[0]), v[1]), v[2]), v[3]);
                }
            } else if (t0 < nb) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool ok = t0 + 4 * g + q < nb;
                        hi[ht] = ok ? fmaxf(hi[ht], e[jl][ht][q]) : hi[ht];
                        lo[ht] = ok ? fminf(lo[ht], e[jl][ht][q]) : lo[ht];
                    }
            }
        }

        // exp2(s - m_p) in place and z_p. exp2f only adjusts arguments below
        // -126 (subnormal results); at or above it, it equals the bare
        // v_exp_f32, which a lane takes unless its scores spread over more
        // than 126 (log2 units).
        bool wide = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            wide = wide || lo[ht] - hi[ht] < -126.0f;
        float z[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            z[ht] = 0.0f;
        auto exp_pass = [&](auto ex) __attribute__((always_inline)) {
#pragma unroll
            for (int jl = 0; jl < JWM; ++jl) {
                const int t0 = 16 * (wave + kWaves * jl);
                if (t0 + 16 <= nb) {
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            e[jl][ht][q] = ex(e[jl][ht][q] - hi[ht]);
                            z[ht] += e[jl][ht][q];
                        }
                } else if (t0 < nb) {
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const bool ok = t0 + 4 * g + q < nb;
                            e[jl][ht][q] = ok ? ex(e[jl][ht][q] - hi[ht]) : 0.0f;
                            z[ht] += e[jl][ht][q];
                        }
                }
            }
        };
        if (wide)
            exp_pass([](float x) __attribute__((always_inline)) { return exp2f(x); });
        else
            exp_pass([](float x) __attribute__((always_inline)) { return __builtin_amdgcn_exp2f(x); });

        // lane partial p = 4 wave + g of head 16 ht + fr (m_p = -inf for a
        // lane without blocks: its factor comes out 0)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int at = (16 * ht + fr) * kPartStride + 4 * wave + g;
            pm[at] = hi[ht];
            pz[at] = z[ht];
        }
        lds_barrier();

        // per head: M, Z and the factors c_p, eight lanes per head with four
        // partials each (the three DPP steps leave the same result in all
        // eight lanes); c_p replaces m_p
        for (int it = tid; it < H * 8; it += kThreads) {
            float *m4 = pm + (it >> 3) * kPartStride + 4 * (it & 7);
            const float *z4 = pz + (it >> 3) * kPartStride + 4 * (it & 7);
            const float m0 = m4[0], m1 = m4[1], m2 = m4[2], m3 = m4[3];
            float M = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
            M = fmaxf(M, dpp<kDppXor1>(M));
            M = fmaxf(M, dpp<kDppXor2>(M));
            M = fmaxf(M, dpp<kDppHalfMirror>(M));
            const float w0 = exp2f(m0 - M), w1 = exp2f(m1 - M), w2 = exp2f(m2 - M),
                        w3 = exp2f(m3 - M);
            float Z = z4[0] * w0 + z4[1] * w1 + z4[2] * w2 + z4[3] * w3;
            Z += dpp<kDppXor1>(Z);
            Z += dpp<kDppXor2>(Z);
            Z += dpp<kDppHalfMirror>(Z);
            // Z >= 1 (the largest partial has w = 1 and z >= 1): the hardware
            // reciprocal (1 ulp) serves
            const float rz = __builtin_amdgcn_rcpf(Z);
            m4[0] = w0 * rz;
            m4[1] = w1 * rz;
            m4[2] = w2 * rz;
            m4[3] = w3 * rz;
        }
        lds_barrier();

        // Q: per block of this lane, the sum over its head tiles of
        // exp2(s - m_p) c_p, then over the 16 head lanes of the tile row by a
        // transposing reduction: each step pairs lane fr with a partner that
        // differs in one more bit (xor 8, then the mirror inside 8 lanes,
        // which flips bit 2, then xor 2 and xor 1), keeps half of its values
        // and adds the partner's copy of them, so lane fr ends with block
        // 4 g + (fr >> 2) of the tile (fr = 4 k + r, r < 4: the same sum).
        float cf[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            cf[ht] = pm[(16 * ht + fr) * kPartStride + 4 * wave + g];
        const bool b3 = fr & 8, b2 = fr & 4;
#pragma unroll
        for (int jl = 0; jl < JWM; ++jl) {
            const int t0 = 16 * (wave + kWaves * jl);
            if (t0 < nb) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] = e[jl][0][q] * cf[0];
#pragma unroll
                    for (int ht = 1; ht < HT; ++ht)
                        v[q] = __builtin_fmaf(e[jl][ht][q], cf[ht], v[q]);
                }
                // bit 3: keep blocks {0, 1} or {2, 3}
                const float k0 = b3 ? v[2] : v[0], s0 = b3 ? v[0] : v[2];
                const float k1 = b3 ? v[3] : v[1], s1 = b3 ? v[1] : v[3];
                const float x0 = k0 + dpp<kDppRor8>(s0), x1 = k1 + dpp<kDppRor8>(s1);
                // bit 2: keep one of the two
                const float k = b2 ? x1 : x0, s = b2 ? x0 : x1;
                float y = k + dpp<kDppHalfMirror>(s);
                y += dpp<kDppXor2>(y);
                y += dpp<kDppXor1>(y);
                if ((fr & 3) == 0)
                    Q[t0 + 4 * g + (fr >> 2)] = y;
            }
        }
    }
    lds_barrier();
    pool_and_select(a, Q, P, K, R, nb, J, scores, out_idx, tid, lane, wave);
}

}  // namespace

int64_t qsa_select_lds_bytes(int64_t H, int64_t Di, int64_t Bcap, int64_t Jcap, int64_t chunk)
{
    const int64_t jcap4 = (Jcap + 3) / 4 * 4;
    return (H + chunk) * (Di * 2 + 16) +
           4 * ((2 * kWaves + 2) * H + 2 * (chunk / 16) * H + (Bcap + 3) / 4 * 4 + jcap4) +
           12 * (jcap4 < kRankMax ? jcap4 : kRankMax);
}

namespace {

typedef void (*SelectKernel)(QsaSelectArgs);

// the compiled fast-path shapes: Di / 32 in {2, 4}, H / 16 in {1, 2, 4, 8},
// column tiles per wavefront in {1, 2, 4} (16 H / 16 x tiles at most)
#define KVRC_SEL_FAST(DK, HT, JWM)                 \
    if (dk == (DK) && ht == (HT) && jwm == (JWM)) \
        return qsa_select_fast_kernel<DK, HT, JWM>;
#define KVRC_SEL_FAST_HT(DK, HT) KVRC_SEL_FAST(DK, HT, 1) KVRC_SEL_FAST(DK, HT, 2) KVRC_SEL_FAST(DK, HT, 4)

SelectKernel fast_select_kernel(int64_t Di, int64_t H, int64_t Bcap)
{
    if (Di % 32 || H % 16 || Bcap < 1)
        return nullptr;
    const int64_t dk = Di / 32, ht = H / 16;
    const int64_t per_wave = ((Bcap + 15) / 16 + kWaves - 1) / kWaves;
    const int64_t jwm = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : 0;
    KVRC_SEL_FAST_HT(2, 1) KVRC_SEL_FAST_HT(2, 2) KVRC_SEL_FAST_HT(2, 4)
    KVRC_SEL_FAST(2, 8, 1) KVRC_SEL_FAST(2, 8, 2)
    KVRC_SEL_FAST_HT(4, 1) KVRC_SEL_FAST_HT(4, 2) KVRC_SEL_FAST_HT(4, 4)
    KVRC_SEL_FAST(4, 8, 1) KVRC_SEL_FAST(4, 8, 2)
    return nullptr;
}
#undef KVRC_SEL_FAST_HT
#undef KVRC_SEL_FAST

}  // namespace

bool qsa_select_fast_path(int64_t H, int64_t Di, int64_t Bcap)
{
    return fast_select_kernel(Di, H, Bcap) != nullptr;
}

hipError_t launch_qsa_select(const QsaSelectArgs &a, hipStream_t stream)
{
    SelectKernel k = fast_select_kernel(a.Di, a.H, a.Bcap);
    int64_t lds;
    if (k) {
        const int64_t jcap4 = (a.Jcap + 3) / 4 * 4;
        lds = a.H * (a.Di * 2 + 16) + 4 * (2 * kPartStride * a.H + (a.Bcap + 15) / 16 * 16 + jcap4) +
              12 * (jcap4 < kRankMax ? jcap4 : kRankMax);
    } else {
        k = qsa_select_kernel;
        lds = qsa_select_lds_bytes(a.H, a.Di, a.Bcap, a.Jcap, a.chunk);
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k, dim3((uint32_t)a.N), dim3(kThreads), (uint32_t)lds, stream, a);
    return hipGetLastError();
}

}  // namespace kvrc
