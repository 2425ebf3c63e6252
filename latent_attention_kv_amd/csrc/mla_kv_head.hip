// MLA kv-path head for gfx950 (MI355X): projection GEMM on MFMA with the
// norm / RoPE / paged-cache epilogue fused behind it.
//
// Computes, per token t (aclnnMlaPrologV3WeightNz: the third path,
// c^KV = alpha_kv * RmsNorm(x W^DKV) into the cache, and the fourth path,
// k^R = ROPE(x W^KR) into the other cache; RoPE as Formula (1) interleaveRope
// of aclnnKvRmsNormRopeCache, placement as its PA_BNSD index rule):
//   c      = x[t, :] . W^T                       W = [576, He], rows 0..511
//                                                 W^DKV, rows 512..575 W^KR
//   y      = alpha * ((c[0:512] / sqrt(mean(c[0:512]^2) + eps)) * gamma)
//   kr     = cat(c1, c2) * cos[t] + cat(-c2, c1) * sin[t]   on c[512:576]
//   ckv_cache[slot[t]] = bf16(y), k_cache[slot[t]] = bf16(kr); slot -1 skips
// with float32 accumulation of the bf16 products (no rounding of c before
// the norm).
//
// Design: the projection is a dense contraction (2 * 576 * He flops per
// token), so it runs on the matrix cores (v_mfma_f32_16x16x32_bf16). A
// workgroup owns 128 whole token rows, so the row-wise norm, the RoPE and
// the scatter run on the accumulators without writing c to memory:
//   * 8 wavefronts = 2 (rows) x 4 (columns); wavefront (wm, wn) accumulates
//     rows 64 wm .. +64 and columns 144 wn .. +144 as 4 x 9 tiles of 16 x 16;
//   * K advances 32 at a time: the 128 x 32 slice of x and the 576 x 32 slice
//     of W are staged in LDS (double-buffered, rows padded to 80 bytes so
//     that the 16-byte fragment reads of 16 lanes cover all 64 banks once);
//     the next slice is loaded into registers while the current one feeds
//     the MFMAs;
//   * epilogue: squares of the 512 kv columns are reduced across lanes and
//     wavefronts, the rows are normalised and rotated in registers, staged
//     as bf16 rows in LDS and written with 16-byte stores per cache row.
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;                 // token rows per workgroup
constexpr int kCols = 576;                 // projection outputs (512 + 64)
constexpr int kNorm = 512;
constexpr int kRope = 64;
constexpr int kThreads = 512;              // 8 wavefronts
constexpr int kKt = (int)kMlaHeadK;        // K per stage (one MFMA K)
constexpr int kLdsRow = 80;                // bytes per staged row (64 + 16 pad)
constexpr int kStageA = kRows * kLdsRow;   // 10240
constexpr int kStageB = kCols * kLdsRow;   // 46080
constexpr int kStage = kStageA + kStageB;  // 56320
constexpr int kChunks = (kRows + kCols) * (kKt * 2 / 16);   // 16-byte pieces per stage: 2816
constexpr int kFull = kChunks / kThreads;                          // 5 pieces for every thread
constexpr int kTail = kChunks - kFull * kThreads;                  // + 1 for the first 256
constexpr int kLoadIters = kFull + 1;
static_assert(kTail > 0 && kTail % 64 == 0, "tail pieces fill whole wavefronts");
constexpr int kMt = 4, kNt = 9;            // 16 x 16 tiles per wavefront
// epilogue staging: bf16 rows of 512 (+8 pad) and 64 (+8 pad) values
constexpr int kCkvLds = (kNorm + 8) * 2;   // 1040 bytes per row
constexpr int kKLds = (kRope + 8) * 2;     // 144 bytes per row
constexpr int kLdsBytes = 2 * kStage > kRows * (kCkvLds + kKLds) + 4 * kRows * 4
                              ? 2 * kStage
                              : kRows * (kCkvLds + kKLds) + 4 * kRows * 4;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 p = {v, 0.0f};
    const bf16x2 r = __builtin_convertvector(p, bf16x2);
    return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

__global__ __launch_bounds__(kThreads) void mla_kv_head_kernel(MlaKvHeadArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int64_t T = a.T, He = a.He;

    // ---- global -> register loads of one K slice ------------------------
    // piece q < 512: x row q / 4, 16-byte piece q % 4; else W row (q-512) / 4.
    // Pieces q = tid + 512 i: i < kFull for every thread, i = kFull for the
    // first kTail threads (whole wavefronts). Rows past T read row T-1
    // (valid memory; their results are dropped).
    const uint4 *src[kLoadIters];
    int dst[kLoadIters];
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i) {
        const int q = (i < kFull || tid < kTail) ? tid + i * kThreads : 0;
        const int r = q >> 2, c = q & 3;
        if (r < kRows) {
            int64_t t = row0 + r;
            t = t < T ? t : T - 1;
            src[i] = reinterpret_cast<const uint4 *>(a.x + t * He) + c;
            dst[i] = r * kLdsRow + c * 16;
        } else {
            const int n = r - kRows;
            src[i] = reinterpret_cast<const uint4 *>(a.w + (int64_t)n * He) + c;
            dst[i] = kStageA + n * kLdsRow + c * 16;
        }
    }
    const bool tail = tid < kTail;
    static_assert(kFull == 5, "the staging registers below are spelled out for 5 + 1 pieces");
    uint4 s0, s1, s2, s3, s4, s5;       // named, so that they stay in registers

    f32x4 acc[kMt][kNt];
#pragma unroll
    for (int m = 0; m < kMt; ++m)
#pragma unroll
        for (int n = 0; n < kNt; ++n)
            acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // fragment addresses inside a stage: lane l reads row (l % 16) of its
    // tile, K elements 8 (l / 16) .. +8
    const int fr = lane & 15, fk = (lane >> 4) * 16;
    const int a_off = (64 * wm + fr) * kLdsRow + fk;
    const int b_off = kStageA + (144 * wn + fr) * kLdsRow + fk;

    const int64_t nk = He / kKt;
#define KVRC_LOAD_SLICE(k0)                                                    \
    do {                                                                       \
        const int64_t off_ = (k0) / 8;            /* in 16-byte pieces */      \
        s0 = src[0][off_];                                                     \
        s1 = src[1][off_];                                                     \
        s2 = src[2][off_];                                                     \
        s3 = src[3][off_];                                                     \
        s4 = src[4][off_];                                                     \
        if (tail)                                                              \
            s5 = src[5][off_];                                                 \
    } while (0)
#define KVRC_STORE_SLICE(buf)                                                  \
    do {                                                                       \
        unsigned char *base_ = smem + (buf) * kStage;                          \
        *reinterpret_cast<uint4 *>(base_ + dst[0]) = s0;                       \
        *reinterpret_cast<uint4 *>(base_ + dst[1]) = s1;                       \
        *reinterpret_cast<uint4 *>(base_ + dst[2]) = s2;                       \
        *reinterpret_cast<uint4 *>(base_ + dst[3]) = s3;                       \
        *reinterpret_cast<uint4 *>(base_ + dst[4]) = s4;                       \
        if (tail)                                                              \
            *reinterpret_cast<uint4 *>(base_ + dst[5]) = s5;                   \
    } while (0)
    KVRC_LOAD_SLICE(0);
    KVRC_STORE_SLICE(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk)
            KVRC_LOAD_SLICE((kt + 1) * kKt);
        const unsigned char *base = smem + buf * kStage;
        bf16x8 af[kMt];
#pragma unroll
        for (int m = 0; m < kMt; ++m)
            af[m] = *reinterpret_cast<const bf16x8 *>(base + a_off + m * 16 * kLdsRow);
#pragma unroll
        for (int n = 0; n < kNt; ++n) {
            const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(base + b_off + n * 16 * kLdsRow);
#pragma unroll
            for (int m = 0; m < kMt; ++m)
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bf, acc[m][n], 0, 0, 0);
        }
        if (kt + 1 < nk)
            KVRC_STORE_SLICE(buf ^ 1);
        __syncthreads();
    }
#undef KVRC_LOAD_SLICE
#undef KVRC_STORE_SLICE

    // ---- epilogue -----------------------------------------------------------
    // acc[m][n][j] is c[row][col] with row = 64 wm + 16 m + 4 (lane / 16) + j,
    // col = 144 wn + 16 n + lane % 16.
    float *red = reinterpret_cast<float *>(smem + kRows * (kCkvLds + kKLds));   // [4][128]
    unsigned char *ckv_lds = smem;
    unsigned char *k_lds = smem + kRows * kCkvLds;
    const int lr = (lane >> 4) * 4;                       // first row of this lane in a tile
    const int lc = lane & 15;
    const int ntn = wn < 3 ? kNt : 5;                     // tiles holding kv (not rope) columns
#pragma unroll
    for (int m = 0; m < kMt; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int n = 0; n < kNt; ++n)
                if (n < ntn)
                    s += acc[m][n][j] * acc[m][n][j];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 8, 64);
            if (lc == 0)
                red[wn * kRows + 64 * wm + 16 * m + lr + j] = s;
        }
    __syncthreads();

    const float alpha = a.alpha;
#pragma unroll
    for (int m = 0; m < kMt; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 64 * wm + 16 * m + lr + j;
            const float ss = (red[r] + red[kRows + r]) + (red[2 * kRows + r] + red[3 * kRows + r]);
            const float rms = sqrtf(ss / (float)kNorm + a.eps);
            int64_t t = row0 + r;
            t = t < T ? t : T - 1;
#pragma unroll
            for (int n = 0; n < kNt; ++n) {
                const int col = 144 * wn + 16 * n + lc;
                const float v = acc[m][n][j];
                if (n < ntn) {
                    const float g = bf16_to_f32(a.gamma[col]);
                    const float yv = alpha * ((v / rms) * g);
                    *reinterpret_cast<uint16_t *>(ckv_lds + r * kCkvLds + col * 2) = f32_to_bf16(yv);
                } else {
                    // rope column m2 = col - 512: pair i = m2 / 2; the partner
                    // of an even column is the next lane and vice versa
                    const int m2 = col - kNorm;
                    const float p = __shfl_xor(v, 1, 64);
                    const int i = m2 >> 1;
                    const bool odd = m2 & 1;
                    const int o = odd ? kRope / 2 + i : i;
                    const float cs = bf16_to_f32(a.cos[t * kRope + o]);
                    const float sn = bf16_to_f32(a.sin[t * kRope + o]);
                    const float kr = odd ? v * cs + p * sn : v * cs - p * sn;
                    *reinterpret_cast<uint16_t *>(k_lds + r * kKLds + o * 2) = f32_to_bf16(kr);
                }
            }
        }
    __syncthreads();

    // ---- scatter: wavefront w writes rows w, w + 8, ... ---------------------
    for (int r = wave; r < kRows; r += kThreads / 64) {
        const int64_t t = row0 + r;
        if (t >= T)
            break;
        const int64_t v = a.slot[t];
        if (v < 0 || v >= a.cache_rows) {
            if (v != -1 && lane == 0 && a.err)
                atomicAdd(a.err, 1);
            continue;
        }
        const uint4 cv = *reinterpret_cast<const uint4 *>(ckv_lds + r * kCkvLds + lane * 16);
        *reinterpret_cast<uint4 *>(a.ckv_cache + v * kNorm + lane * 8) = cv;
        if (lane < 8) {
            const uint4 kv = *reinterpret_cast<const uint4 *>(k_lds + r * kKLds + lane * 16);
            *reinterpret_cast<uint4 *>(a.k_cache + v * kRope + lane * 8) = kv;
        }
    }
}

}  // namespace

hipError_t launch_mla_kv_head(const MlaKvHeadArgs &a, hipStream_t stream)
{
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    const int64_t grid = (a.T + kRows - 1) / kRows;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(mla_kv_head_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(mla_kv_head_kernel, dim3((uint32_t)grid), dim3(kThreads), kLdsBytes, stream,
                       a);
    return hipGetLastError();
}

}  // namespace kvrc
