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
//            (evaluated as (c * (1 / rms)) * (alpha * gamma): float32 steps
//            of their own, within the derived bound like the projection)
//   kr     = cat(c1, c2) * cos[t] + cat(-c2, c1) * sin[t]   on c[512:576]
//   ckv_cache[slot[t]] = bf16(y), k_cache[slot[t]] = bf16(kr); slot -1 skips
//   (slot[t] from a per-token slot mapping, or from one block-index entry
//   per chunk of BlockSize tokens of a sequence: PA_BLK_BSND)
//   or, for a quantised ckv cache (the per-row rule of the norm-rope-cache
//   operator: scale = RowMax(|y|) / 127 with rounded int8 codes, or
//   RowMax(|y|) / 448 with the nearest FLOAT8 E4M3FN codes),
//   ckv_cache[slot[t]] = codes of y * RN(1 / scale), ckv_scale[slot[t]] = scale,
//   with RowMax(|y|) taken as (1 / rms) * max |c * alpha * gamma| (equal to
//   the maximum of the rounded y up to a few roundings)
// with float32 accumulation of the bf16 products (no rounding of c before
// the norm).
//
// Design: the projection is a dense contraction (2 * 576 * He flops per
// token), so it runs on the matrix cores (v_mfma_f32_16x16x32_bf16). The
// operands reach a compute unit through its texture path, whose rate bounds
// this kernel, so the tile is chosen for bytes per flop: a PAIR of
// workgroups owns 256 token rows, one workgroup per half of the 576 output
// columns (columns 0..287, and 288..575 with the 64 rope columns). Per 32
// of K a workgroup then streams 16 KiB of x and 18 KiB of W (34 KiB)
// instead of 8 + 36 KiB for a 128 x 576 tile, for the same matrix work.
//   * 8 wavefronts = 4 (rows) x 2 (columns); wavefront (wm, wn) accumulates
//     rows 64 wm .. +64 and columns 144 wn .. +144 of its half as 4 x 9 tiles
//     of 16 x 16 (144 accumulator registers, two wavefronts per SIMD);
//   * K advances 64 at a time (two MFMA steps of 32): a staged row is then
//     one whole 128-byte line of x or W, which halves the line requests per
//     byte against 64-byte rows (measured: ~5 % of the call); the slices pass
//     through two LDS rings filled by direct global -> LDS loads
//     (global_load_lds_dwordx4: no staging registers, no LDS store
//     instructions), W (288 x 64, 36 KiB) and x (256 x 64, 32 KiB), two
//     stages each, loaded one step ahead of the MFMAs; each wavefront waits
//     only for its own loads, then one barrier publishes them;
//   * the two workgroups of a pair are blockIdx b and b + 8, which the
//     dispatcher places on the same XCD: their x rows meet in that XCD's L2;
//   * staged rows are 128 bytes with their eight 16-byte pieces permuted
//     (swz below) so that every eight lanes of a fragment read, which the
//     LDS serves together, hit eight different 16-byte bank groups;
//   * epilogue: the MFMAs take W as their first operand, so each lane's
//     accumulators are 4 consecutive output columns of one token row (no
//     transpose); squares are reduced per row across lanes (permlane swaps)
//     and wavefronts; the two workgroups of the pair swap
//     their per-row partial sums through the caller's workspace (a ready
//     flag per half, set after the sums; the partner reads the sums, zeroes
//     them and clears the flag, so the workspace is all zero again when the
//     call ends; see the claim protocol below);
//     rows are normalised and rotated in registers, staged as bf16 in LDS
//     and scattered with 16-byte stores per cache row piece;
//   * a quantised ckv cache needs the maximum of each row over both halves:
//     each half takes its partial maximum of |c * alpha * gamma| with its
//     square sums, and both travel through the one exchange (a second area
//     of the workspace); the normalised values stay in the accumulator
//     registers until the scale is known, then the codes are staged (one
//     byte each) and scattered like the bf16 rows, half 0 also writing the
//     row scale.
// No wait depends on the two halves of a pair being resident together (HIP
// promises nothing about dispatch order or co-residency): each half claims
// its half of the pair in the workspace when it starts (a claim word per
// half, marked with a tag fresh for every call). A half that reaches the
// exchange and finds neither its partner's partials nor its partner's claim
// after a short wait claims the partner's half itself ("takeover") and
// computes both halves, one after the other with the same code, so the
// outputs are the same bits; the partner, when it is placed, finds its half
// taken and leaves without writing. A partner that has claimed is resident
// and running, so waiting for its partials always ends (a bound of seconds
// only keeps the kernel finite). Two calls may run at the same time on one
// device, each with its own workspace.
#include <atomic>

#include "device_common.hpp"
#include "kvrc_launch.hpp"

namespace kvrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRows = (int)kMlaPairRows;   // token rows per workgroup pair
constexpr int kHalfCols = 288;             // output columns per workgroup
constexpr int kNorm = 512;
constexpr int kRope = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKt = (int)kMlaHeadK;        // K of one MFMA (32)
constexpr int kKs = 2 * kKt;               // K per ring stage (64): a staged row is
                                           // one 128-byte line of x or W
constexpr int kRowBytes = kKs * 2;         // 128
constexpr int kStageA = kRows * kRowBytes; // 32768
constexpr int kStageB = kHalfCols * kRowBytes; // 36864
// Two LDS rings of two stages each, W slices and x slices, each stage loaded
// one step (K 64) ahead of its MFMAs.
constexpr int kWStages = 2, kXStages = 2;
constexpr int kXRing = kWStages * kStageB;              // offset of the x ring
constexpr int kPipeBytes = kXRing + kXStages * kStageA; // 139264
// the 32 x blocks and 36 W blocks (1 KiB = 8 rows each, one load
// instruction) of a stage: wavefront w loads x blocks 4w .. 4w + 3, then W
// blocks (5 each for w < 4, 4 for the others)
constexpr int kXBlocks = 4;
static_assert(kStageA / 1024 == kXBlocks * kWaves && 4 * 5 + 4 * 4 == kStageB / 1024,
              "block split");
constexpr int kMaxWBlocks = 5;
constexpr int kMt = 4, kNt = 9;            // 16 x 16 tiles per wavefront
constexpr int kWaveCols = kNt * 16;        // 144
constexpr int kRopeTiles = 4;              // tiles 5..8 of the rope wavefront
// epilogue staging: bf16 rows of 288 (+8 pad) values, then the per-column-
// wavefront square sums and the full square sums per row
constexpr int kStageRow = (kHalfCols + 8) * 2;   // 592 bytes per row
constexpr int kRedOff = kRows * kStageRow;
constexpr int kSumOff = kRedOff + 2 * kRows * 4;
// quantised ckv: per-column-wavefront partial row maxima, then the row maxima
constexpr int kRedMaxOff = kSumOff + kRows * 4;
constexpr int kMaxOff = kRedMaxOff + 2 * kRows * 4;
constexpr int kEpiBytes = kMaxOff + kRows * 4;
// two control words (the claim result, the exchange outcome), after both
constexpr int kCtlOff = kPipeBytes > kEpiBytes ? kPipeBytes : kEpiBytes;
constexpr int kLdsBytes = kCtlOff + 16;
// Claim words of the workspace: the call tag times 4 plus a state.
constexpr uint32_t kClaimed = 1, kStolen = 2;
// Outcomes of a pass's exchange step.
constexpr int kGot = 0, kStole = 1, kLost = 2, kExit = 3;
// Wall-clock (100 MHz) bound of a wait for a partner that has claimed its
// half: such a partner is resident and running, so its partials come; the
// bound (10 s) only keeps the kernel finite.
constexpr uint64_t kSafetyTicks = 1000000000ull;
// cache-policy operand of a buffer store: sc1 (device scope, write-through)
constexpr int kStoreSc1 = 16;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; the unused counters at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Piece permutation of a staged row (128 bytes, eight 16-byte pieces): piece
// c of row r sits in slot c ^ (r % 8). The LDS serves a 16-byte read eight
// lanes (128 bytes) at a time; the eight lanes of a fragment read take rows
// r .. r + 7 (r a multiple of 8) at one piece, so they hit eight different
// slots, i.e. eight different 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return r & 7; }

// Claim of a half, in two steps by wavefront 0, lane 0. At the start,
// claim_begin reads this half's flag and tries the claim word from 0 to this
// call's "claimed" (the results are read only after the K loop, so the
// atomics' latency hides behind it). After the K loop, claim_settle tells
// whether the partner took the half over: then both words of this half are
// reset to zero (nobody else touches them again in this call). A word that
// was neither zero nor this call's (left by another call: a workspace that
// was not zero) is counted in err, and the claim is retried from it.
struct ClaimStart {
    uint32_t old_claim, old_flag;
};

__device__ __forceinline__ ClaimStart claim_begin(uint32_t *my_claim, const uint32_t *my_flag,
                                                  uint32_t tag)
{
    ClaimStart c;
    c.old_flag = __hip_atomic_load(my_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t expected = 0u;
    __hip_atomic_compare_exchange_strong(my_claim, &expected, (tag << 2) | kClaimed,
                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    c.old_claim = expected;                 // 0 when the claim succeeded
    return c;
}

__device__ bool claim_settle(ClaimStart c, uint32_t *my_claim, uint32_t *my_flag, uint32_t tag,
                             int32_t *err)
{
    const uint32_t claimed = (tag << 2) | kClaimed, stolen = (tag << 2) | kStolen;
    // the raw values are first looked at here (the compiler may not move a
    // comparison of them, and with it the wait for the atomics, before the
    // K loop)
    asm volatile("" : "+v"(c.old_flag), "+v"(c.old_claim));
    bool dirty = c.old_flag != 0u;
    bool taken = c.old_claim == stolen;
    if (c.old_claim != 0u && !taken) {
        dirty = true;
        uint32_t old = c.old_claim;
        for (;;) {             // a failed exchange means the partner just took it
            if (old == stolen) {
                taken = true;
                break;
            }
            uint32_t expected = old;
            if (__hip_atomic_compare_exchange_strong(my_claim, &expected, claimed,
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                break;
            old = expected;
        }
    }
    if (taken) {               // this half's words are no one else's any more
        __hip_atomic_store(my_claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(my_flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (dirty && err)
        atomicAdd(err, 1);
    return taken;
}

// The exchange of per-row partial values between the two workgroups of a
// pair, run by wavefront 0 (lane l: rows 4 l .. 4 l + 3): publish p (and p2,
// with kTwo) in this half's areas of the workspace, then the flag (this
// call's tag, with release order); wait for the partner's flag. Outcomes:
//   kGot   - the partner's values are in q (q2); their areas are zeroed, its
//            flag cleared and its claim word reset (the partner touches
//            neither again in this call);
//   kStole - the partner did not publish within steal_ticks and had not
//            claimed its half: this workgroup claimed it instead ("stolen")
//            and computes both halves; the partner, when it starts, sees the
//            word and leaves;
//   kLost  - the partner claimed its half but published nothing within the
//            safety bound (not expected while the GPU makes progress).
// A partner that has claimed its half is resident and running, so waiting
// for it always ends; a partner that has not is never waited for beyond
// steal_ticks. No wait depends on the dispatch order or on co-residency.
template <bool kTwo>
__device__ __forceinline__ int pair_exchange(float *mine, float *theirs, float *mine2,
                                             float *theirs2, uint32_t *my_flag,
                                             uint32_t *their_flag, uint32_t *their_claim,
                                             uint32_t tag, uint32_t steal_ticks,
                                             const float (&p)[4], const float (&p2)[4],
                                             float (&q)[4], float (&q2)[4], int lane)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        __hip_atomic_store(mine + 4 * lane + j, p[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kTwo)
            __hip_atomic_store(mine2 + 4 * lane + j, p2[j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    // release: the wavefront's values above are visible before the flag
    if (lane == 0)
        __hip_atomic_store(my_flag, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int outcome = kGot;
    if (lane == 0) {
        const uint32_t claimed = (tag << 2) | kClaimed, stolen = (tag << 2) | kStolen;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool tried = false;
        for (;;) {
            if (__hip_atomic_load(their_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag)
                break;
            const uint64_t waited = __builtin_amdgcn_s_memrealtime() - t0;
            if (!tried && waited >= steal_ticks) {
                tried = true;
                uint32_t c = __hip_atomic_load(their_claim, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                while (c != claimed) {
                    uint32_t expected = c;
                    if (__hip_atomic_compare_exchange_strong(their_claim, &expected, stolen,
                                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)) {
                        outcome = kStole;
                        break;
                    }
                    c = expected;
                }
                if (outcome == kStole)
                    break;
            }
            if (waited >= kSafetyTicks) {
                outcome = kLost;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    outcome = __builtin_amdgcn_readfirstlane(outcome);
    if (outcome != kGot)
        return outcome;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[j] = __hip_atomic_load(theirs + 4 * lane + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(theirs + 4 * lane + j, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kTwo) {
            q2[j] = __hip_atomic_load(theirs2 + 4 * lane + j, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(theirs2 + 4 * lane + j, 0.0f, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the partner's values are read and zeroed, and it has published its
    // last word for this call: clear its flag and its claim
    if (lane == 0) {
        __hip_atomic_store(their_flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(their_claim, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return kGot;
}

// Q: the ckv cache type (kvrc_cache_dtype: 0 bf16, 1 int8, 2 E4M3FN).
// steal_ticks, stall_ticks: a.steal_us, a.stall_us in ticks of the device's
// wall clock (s_memrealtime).
template <int Q>
__global__ __launch_bounds__(kThreads)
void mla_kv_head_kernel(MlaKvHeadArgs a, uint32_t steal_ticks, uint32_t stall_ticks)
{
    constexpr int kEsz = Q == 0 ? 2 : 1;        // bytes per ckv element
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int wm = wave & 3, wn = wave >> 2;
    const int nw = wave < 4 ? 5 : 4;                     // W blocks of this wavefront
    const int wb0 = wave < 4 ? 5 * wave : 20 + 4 * (wave - 4);
    // blockIdx b and b + 8 form a pair (same XCD under round-robin dispatch)
    const int bx = blockIdx.x;
    const int half = (bx >> 3) & 1;
    const int64_t pair = (int64_t)(bx >> 4) * 8 + (bx & 7);
    const int64_t T = a.T, He = a.He;
    const int64_t npairs = (T + kRows - 1) / kRows;
    if (pair >= npairs)
        return;                               // padding of the grid: both halves leave
    const int64_t row0 = pair * kRows;

    // ---- workspace: float sums[npairs][2][256], float maxima[npairs][2][256]
    // (quantised ckv only), uint32 flags[npairs][2], uint32 claims[npairs][2]
    float *const part = reinterpret_cast<float *>(a.workspace);
    uint32_t *const flags = reinterpret_cast<uint32_t *>(part + npairs * 4 * kRows);
    uint32_t *const claims = flags + npairs * 2;
    auto area = [&](int k, int h) { return part + ((k * npairs + pair) * 2 + h) * kRows; };
    uint32_t *const ctl = reinterpret_cast<uint32_t *>(smem + kCtlOff);

    // ---- claim this half for the call (settled after the first K loop) ----
    // (left unset outside wavefront 0, lane 0, the only lane that reads it:
    // no merge of values at the end of the branch, which would wait for the
    // atomics here)
    ClaimStart claim;
    if (wave == 0 && lane == 0) {
        if (half == 1 && stall_ticks) {                 // test only
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__builtin_amdgcn_s_memrealtime() - t0 < stall_ticks)
                __builtin_amdgcn_s_sleep(8);
        }
        claim = claim_begin(claims + pair * 2 + half, flags + pair * 2 + half, a.tag);
    }

    // Passes: 0 = this half, its partials exchanged with the partner; after a
    // takeover (kStole) 1 = the partner's half, then 2 = this half again
    // (the accumulators hold one half at a time). Every pass runs the same
    // code on the same operands, so a half's outputs are the same bits
    // whichever workgroup computes them.
    auto run_pass = [&](const int hh, const int pass) __attribute__((always_inline)) -> int {
    // Each copy of the pass forms its per-lane values from its own reading
    // of the lane index, so that the copy after a takeover neither shares
    // nor prolongs the registers of the first.
    int lane_v = tid & 63;
    asm volatile("" : "+v"(lane_v));
    const int lane = lane_v;
    // The cache slots of the rows this wavefront scatters (rows wave + 8 i,
    // i < 32) are fetched now, lane i holding row i's: their latency hides
    // behind the K loop instead of preceding each row's stores. With the
    // block-indexed placement the slot of token t = b*S + s is
    // (entry / BS) * BS + s % BS for the entry of its chunk s / BS; an
    // entry outside [-1, rows) becomes -2 (counted in the scatter).
    int64_t my_slot = -1;
    {
        const int64_t t = row0 + wave + kWaves * (lane & 31);
        if (lane < kRows / kWaves && t < T) {
            if (a.block_index) {
                const int64_t b = t / a.S, s = t - b * a.S;
                const int64_t e = a.block_index[b * a.chunks + s / a.block_size];
                my_slot = e == -1 ? -1
                        : (e < -1 || e >= a.cache_rows) ? -2
                        : (e / a.block_size) * a.block_size + s % a.block_size;
            } else {
                my_slot = a.slot[t];
            }
        }
    }
    unsigned char *const xdst = smem + kXRing + wave * kXBlocks * 1024;  // + stage * kStageA
    unsigned char *const wdst = smem + wb0 * 1024;               // + stage * kStageB + i KiB

    const bool rope_wave = hh == 1 && wn == 1;           // columns 432..575 of the output
    const int ntn = rope_wave ? kNt - kRopeTiles : kNt;  // tiles holding kv (not rope) columns
    // ---- direct global -> LDS loads ---------------------------------------
    // A 1 KiB block holds 8 rows of 128 bytes (one stage); lane l writes
    // byte 16 l: row 8 b + l / 8, slot l % 8, i.e. piece (l % 8) ^ (l / 8) of
    // that row. x block b = token rows 8 b .. +8 (rows past T read row T - 1:
    // valid memory, results dropped); W block b = rows 8 b .. +8 of the
    // pass's half of W. When He = 64 q + 32, the last stage holds K 0..31
    // only: its lanes of pieces 4..7 reread their row's pieces 0..3 (within
    // the row), and its second MFMA step is skipped.
    const int piece = (lane & 7) ^ (lane >> 3);
    const uint16_t *xsrc[kXBlocks];
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i) {
        const int r = 8 * (kXBlocks * wave + i) + (lane >> 3);
        int64_t t = row0 + r;
        t = t < T ? t : T - 1;
        xsrc[i] = a.x + t * He + piece * 8;
    }
    const uint16_t *wsrc[kMaxWBlocks];
#pragma unroll
    for (int i = 0; i < kMaxWBlocks; ++i) {
        const int r = (wb0 + (i < nw ? i : 0)) * 8 + (lane >> 3);
        wsrc[i] = a.w + (int64_t)(kHalfCols * hh + r) * He + piece * 8;
    }
    const int nks = (int)((He + kKs - 1) / kKs);
    const bool tail = He % kKs != 0;                     // He % 64 == 32
    const int tail_back = tail && piece >= 4 ? kKt : 0;

    f32x4 acc[kMt][kNt];
#pragma unroll
    for (int m = 0; m < kMt; ++m)
#pragma unroll
        for (int n = 0; n < kNt; ++n)
            acc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // fragment reads: lane l takes row (l % 16) of a tile, K piece l / 16 of
    // the MFMA step's 32 (piece 4 s + l / 16 of the staged row in step s);
    // tile row offsets are multiples of 16, so swz of the row is swz(l % 16)
    const int fr = lane & 15, fc = lane >> 4;
    int a_off[2], b_off[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        a_off[sb] = (64 * wm + fr) * kRowBytes + (((4 * sb + fc) ^ swz(fr)) << 4);
        b_off[sb] = (kWaveCols * wn + fr) * kRowBytes + (((4 * sb + fc) ^ swz(fr)) << 4);
    }

    // prologue: stage 0, x then W
    {
        const int back = nks == 1 ? tail_back : 0;
#pragma unroll
        for (int i = 0; i < kXBlocks; ++i)
            __builtin_amdgcn_global_load_lds(xsrc[i] - back, (lds_void *)(xdst + i * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < kMaxWBlocks; ++i)
            if (i < nw)
                __builtin_amdgcn_global_load_lds(wsrc[i] - back, (lds_void *)(wdst + i * 1024), 16, 0,
                                                 0);
    }
    for (int ks = 0; ks < nks; ++ks) {
        // Every load of this wavefront still in flight is for stage ks
        // (issued during step ks - 1, or the prologue); the barrier then
        // publishes every wavefront's and tells that all are past step
        // ks - 1, whose buffers are refilled during this step.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // raised wave priority while this step's MFMAs issue (the arbiter
        // favours the wavefront feeding the matrix pipe)
        __builtin_amdgcn_s_setprio(1);
        const int sn = ks + 1;                           // the stage loaded during this step
        const bool more = sn < nks;
        const int64_t koff = (int64_t)sn * kKs - (sn == nks - 1 ? tail_back : 0);
        unsigned char *const xd = xdst + (sn & 1) * kStageA;
        unsigned char *const wd = wdst + (sn & 1) * kStageB;
        const unsigned char *xbase = smem + kXRing + (ks & 1) * kStageA;
        const unsigned char *wbase = smem + (ks & 1) * kStageB;
        const int nsub = tail && ks == nks - 1 ? 1 : 2;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            if (sb == 1 && nsub == 1)
                break;
            bf16x8 af[kMt], bf[2];
#pragma unroll
            for (int m = 0; m < kMt; ++m)
                af[m] = *reinterpret_cast<const bf16x8 *>(xbase + a_off[sb] + m * 16 * kRowBytes);
            bf[0] = *reinterpret_cast<const bf16x8 *>(wbase + b_off[sb]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < kNt; ++n) {
                if (n + 1 < kNt)
                    bf[(n + 1) & 1] =
                        *reinterpret_cast<const bf16x8 *>(wbase + b_off[sb] + (n + 1) * 16 * kRowBytes);
                // during the first MFMA step, one load between MFMA groups:
                // the x blocks first, then W
                if (sb == 0 && more) {
                    if (n < kXBlocks) {
                        __builtin_amdgcn_global_load_lds(xsrc[n] + koff, (lds_void *)(xd + n * 1024),
                                                         16, 0, 0);
                    } else if (n - kXBlocks < kMaxWBlocks) {
                        if (n - kXBlocks < nw)
                            __builtin_amdgcn_global_load_lds(wsrc[n - kXBlocks] + koff,
                                                             (lds_void *)(wd + (n - kXBlocks) * 1024),
                                                             16, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < kMt; ++m)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[n & 1], af[m], acc[m][n], 0,
                                                                        0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();                          // every stage read: LDS reused below

    // ---- epilogue -----------------------------------------------------------
    // The MFMAs take the W fragment as their first operand, so a tile is
    // c^T: acc[m][n][e] is c[row][col] with
    //   row = 64 wm + 16 m + lane % 16,
    //   col = 288 half + 144 wn + 16 n + 4 (lane / 16) + e,
    // four consecutive columns of one token row in each lane.
    const int rsub = lane & 15;                          // row within a 16-row tile
    const int cq = 4 * (lane >> 4);                      // first column within a tile
    // The rope tiles (rope wavefront, tiles 5..8) need the cos / sin pairs
    // (i0, i0 + 1) and (32 + i0, 33 + i0), i0 = 8 (n - 5) + cq / 2: those of
    // row tile 0 are loaded now, those of row tile m + 1 while row tile m is
    // computed (two register buffers), so their latencies overlap work.
    uint32_t rc[2][kRopeTiles][4];
    auto load_rope_tables = [&](int m, uint32_t (&dst)[kRopeTiles][4]) {
        int64_t t = row0 + 64 * wm + 16 * m + rsub;
        t = t < T ? t : T - 1;
#pragma unroll
        for (int k = 0; k < kRopeTiles; ++k) {
            const int i0 = 8 * k + cq / 2;
            dst[k][0] = *reinterpret_cast<const uint32_t *>(a.cos + t * kRope + i0);
            dst[k][1] = *reinterpret_cast<const uint32_t *>(a.cos + t * kRope + 32 + i0);
            dst[k][2] = *reinterpret_cast<const uint32_t *>(a.sin + t * kRope + i0);
            dst[k][3] = *reinterpret_cast<const uint32_t *>(a.sin + t * kRope + 32 + i0);
        }
    };
    if (rope_wave)
        load_rope_tables(0, rc[0]);
    float *red = reinterpret_cast<float *>(smem + kRedOff);     // [2 column wavefronts][256]
    float *sums = reinterpret_cast<float *>(smem + kSumOff);    // [256]
    float *red_max = reinterpret_cast<float *>(smem + kRedMaxOff);  // [2][256] (quantised)
    float *maxs = reinterpret_cast<float *>(smem + kMaxOff);        // [256] (quantised)
    // alpha_kv * gamma per column, once: each output is then two products,
    // (c * rr) * (alpha * gamma)
    const float alpha = a.alpha;
    float g[kNt][4];
#pragma unroll
    for (int n = 0; n < kNt; ++n) {
        const int col = kHalfCols * hh + kWaveCols * wn + 16 * n + cq;
        const uint2 gw = *reinterpret_cast<const uint2 *>(a.gamma + (col < kNorm ? col : 0));
        g[n][0] = alpha * bf16_lo(gw.x); g[n][1] = alpha * bf16_hi(gw.x);
        g[n][2] = alpha * bf16_lo(gw.y); g[n][3] = alpha * bf16_hi(gw.y);
    }
#pragma unroll
    for (int m = 0; m < kMt; ++m) {
        float s = 0.0f;
        float mx = 0.0f;                     // max |c * alpha * gamma| (quantised ckv)
#pragma unroll
        for (int n = 0; n < kNt; ++n)
            if (n < ntn)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s += acc[m][n][e] * acc[m][n][e];
                    if constexpr (Q != 0)
                        mx = fmaxf(mx, fabsf(acc[m][n][e] * g[n][e]));
                }
        // add the four column quarters (lanes l, l ^ 16, l ^ 32, l ^ 48): a
        // permlane swap of the value with itself leaves the two halves of
        // the exchange in its two results, in every lane
        {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s),
                                                              false, false);
            s = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s),
                                                              false, false);
            s = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        }
        if constexpr (Q != 0) {
            const auto m16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                              false, false);
            mx = fmaxf(__uint_as_float(m16[0]), __uint_as_float(m16[1]));
            const auto m32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                              false, false);
            mx = fmaxf(__uint_as_float(m32[0]), __uint_as_float(m32[1]));
            if (cq == 0)
                red_max[wn * kRows + 64 * wm + 16 * m + rsub] = mx;
        }
        if (cq == 0)
            red[wn * kRows + 64 * wm + 16 * m + rsub] = s;
    }
    __syncthreads();

    // ---- the per-row partials of both halves ------------------------------
    if (wave == 0) {
        float p[4], q[4], p2[4], q2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = red[4 * lane + j] + red[kRows + 4 * lane + j];
            p2[j] = Q != 0 ? fmaxf(red_max[4 * lane + j], red_max[kRows + 4 * lane + j]) : 0.0f;
        }
        int st = kGot;
        if (pass == 0) {
            bool taken = false;
            if (lane == 0)
                taken = claim_settle(claim, claims + pair * 2 + half, flags + pair * 2 + half,
                                     a.tag, a.err);
            if (__builtin_amdgcn_readfirstlane((int)taken)) {
                st = kExit;            // the partner took this half over
            } else {
                st = pair_exchange<Q != 0>(area(0, hh), area(0, 1 - hh), area(1, hh),
                                           area(1, 1 - hh), flags + pair * 2 + hh,
                                           flags + pair * 2 + (1 - hh),
                                           claims + pair * 2 + (1 - hh), a.tag, steal_ticks,
                                           p, p2, q, q2, lane);
                if (st == kStole && lane == 0 && a.steals)
                    atomicAdd(a.steals, 1);
                if (st == kLost && lane == 0 && a.err)
                    atomicAdd(a.err, 1);
            }
        } else {
            // after a takeover both areas of the pair are this workgroup's:
            // pass 1 keeps the partner's partials in the partner's areas,
            // next to this half's, published in pass 0 (each lane rereads
            // only the rows it wrote)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (pass == 1) {
                    __hip_atomic_store(area(0, hh) + 4 * lane + j, p[j], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    if constexpr (Q != 0)
                        __hip_atomic_store(area(1, hh) + 4 * lane + j, p2[j], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                q[j] = __hip_atomic_load(area(0, 1 - hh) + 4 * lane + j, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
                q2[j] = Q != 0 ? __hip_atomic_load(area(1, 1 - hh) + 4 * lane + j,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0.0f;
            }
        }
        if (st == kGot) {
            // the same order in both halves: the sum of columns 0..287 first
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sums[4 * lane + j] = hh == 0 ? p[j] + q[j] : q[j] + p[j];
                if constexpr (Q != 0)
                    maxs[4 * lane + j] = fmaxf(p2[j], q2[j]);
            }
        }
        if (lane == 0)
            ctl[1] = (uint32_t)st;
    }
    __syncthreads();
    const int outcome = (int)ctl[1];
    if (outcome != kGot)
        return outcome;                       // nothing written by this pass

    unsigned char *stage = smem;
    // 1 / rms of row r (the same expression wherever it is needed) and, for a
    // quantised ckv cache, the row scale RN(RN(rr * max |c alpha gamma|) / d)
    auto row_rr = [&](int r) { return 1.0f / sqrtf(sums[r] / (float)kNorm + a.eps); };
    constexpr float kDiv = Q == 1 ? 127.0f : kE4m3Max;
    auto row_scale_of = [&](int r) { return row_scale(row_rr(r) * maxs[r], kDiv); };
#pragma unroll
    for (int m = 0; m < kMt; ++m) {
        if (rope_wave && m + 1 < kMt)
            load_rope_tables(m + 1, rc[(m + 1) & 1]);
        const int r = 64 * wm + 16 * m + rsub;
        const float rr = row_rr(r);
#pragma unroll
        for (int n = 0; n < kNt; ++n) {
            const f32x4 v = acc[m][n];
            if (n < ntn) {
                const int col = kWaveCols * wn + 16 * n + cq;       // within the half
                const f32x4 y = {(v[0] * rr) * g[n][0], (v[1] * rr) * g[n][1],
                                 (v[2] * rr) * g[n][2], (v[3] * rr) * g[n][3]};
                if constexpr (Q == 0) {
                    const uint2 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
                    *reinterpret_cast<uint2 *>(stage + r * kStageRow + col * 2) = o;
                } else {
                    acc[m][n] = y;           // coded below, with the row scale
                }
            } else {
                // rope columns 2 i0 .. 2 i0 + 3 of c[512:]: pairs (2 i0, 2 i0 + 1)
                // and (2 i0 + 2, 2 i0 + 3) give outputs i0, i0 + 1 and
                // 32 + i0, 33 + i0, staged after the 224 kv columns of the half
                const int k = n - ntn > 0 ? n - ntn : 0;   // n >= ntn here
                const int i0 = 8 * k + cq / 2;
                const uint32_t c0 = rc[m & 1][k][0], c1 = rc[m & 1][k][1];
                const uint32_t s0 = rc[m & 1][k][2], s1 = rc[m & 1][k][3];
                const float lo0 = v[0] * bf16_lo(c0) - v[1] * bf16_lo(s0);
                const float lo1 = v[2] * bf16_hi(c0) - v[3] * bf16_hi(s0);
                const float hi0 = v[1] * bf16_lo(c1) + v[0] * bf16_lo(s1);
                const float hi1 = v[3] * bf16_hi(c1) + v[2] * bf16_hi(s1);
                unsigned char *kr = stage + r * kStageRow + (kNorm - kHalfCols) * kEsz;
                *reinterpret_cast<uint32_t *>(kr + i0 * 2) = pack_bf16x2(lo0, lo1);
                *reinterpret_cast<uint32_t *>(kr + (32 + i0) * 2) = pack_bf16x2(hi0, hi1);
            }
        }
    }
    __syncthreads();

    if constexpr (Q != 0) {
        // ---- code the rows ------------------------------------------------
#pragma unroll
        for (int m = 0; m < kMt; ++m) {
            const int r = 64 * wm + 16 * m + rsub;
            const float scale = row_scale_of(r);
            // y * RN(1 / scale) in rcp_rn's domain [2^-60, 2^60]; IEEE
            // division outside it (a zero row has scale 0 and codes 0)
            const bool fast = scale >= 0x1p-60f && scale <= 0x1p60f;
            const float rs = fast ? rcp_rn(scale) : 0.0f;
#pragma unroll
            for (int n = 0; n < kNt; ++n) {
                if (n < ntn) {
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        t[e] = fast ? acc[m][n][e] * rs
                                    : (scale > 0.0f ? acc[m][n][e] / scale : 0.0f);
                    uint32_t w;
                    if constexpr (Q == 1) {
                        uint32_t b[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)   // low byte of the bits: rint(t), half even
                            b[e] = __float_as_uint(__builtin_amdgcn_fmed3f(t[e], -127.0f, 127.0f) +
                                                   kRoundMagic);
                        w = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) |
                            __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
                    } else {
                        w = e4m3_pack4(e4m3_clamp(t[0]), e4m3_clamp(t[1]), e4m3_clamp(t[2]),
                                       e4m3_clamp(t[3]));
                    }
                    const int col = kWaveCols * wn + 16 * n + cq;
                    *reinterpret_cast<uint32_t *>(stage + r * kStageRow + col) = w;
                }
            }
        }
        __syncthreads();
    }

    // ---- scatter: wavefront w writes its half of rows w, w + 8, ... --------
    // half 0: ckv bytes [0, 576) of the row (36 pieces of 16 bytes; [0, 288),
    // 18 pieces, for one-byte codes, and the row scale);
    // half 1: ckv bytes [576, 1024) (28 pieces; [288, 512), 14 pieces), then
    // the k row (8 pieces).
    // Caches below 4 GiB take sc1 (device scope) buffer stores, which write
    // through the XCD's L2 instead of leaving the rows dirty there: the
    // write-backs of the swap above and of the kernel's end then find little
    // to flush. The descriptors cover exactly the caches.
    constexpr int kCkvPieces0 = kHalfCols * kEsz / 16;           // 36 (18)
    constexpr int kCkvPieces1 = (kNorm - kHalfCols) * kEsz / 16;  // 28 (14)
    constexpr int kKPieces = kRope * 2 / 16;                      // 8
    const int nckv = hh == 0 ? kCkvPieces0 : kCkvPieces1;
    const int npieces = hh == 0 ? kCkvPieces0 : kCkvPieces1 + kKPieces;
    const int64_t ckv_row = kNorm * kEsz;
    const bool buf = a.cache_rows * ckv_row <= (int64_t)UINT32_MAX;
    const __amdgpu_buffer_rsrc_t ckv_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.ckv_cache, 0, (int)(uint32_t)(a.cache_rows * ckv_row),
                                          0x00020000);
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.k_cache, 0, (int)(uint32_t)(a.cache_rows * kRope * 2),
                                          0x00020000);
#pragma unroll 4
    for (int i = 0; i < kRows / kWaves; ++i) {
        const int r = wave + kWaves * i;
        const int64_t t = row0 + r;
        if (t >= T)
            break;
        const int64_t v = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                         (int)(my_slot >> 32), i) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)my_slot, i));
        if (v < 0 || v >= a.cache_rows) {
            if (hh == 0 && v != -1 && lane == 0 && a.err)
                atomicAdd(a.err, 1);
            continue;
        }
        if constexpr (Q != 0) {
            if (hh == 0 && lane == 63)
                a.ckv_scale[v] = row_scale_of(r);
        }
        if (lane < npieces) {
            const uint4 cv = *reinterpret_cast<const uint4 *>(stage + r * kStageRow + lane * 16);
            const u32x4 w = {cv.x, cv.y, cv.z, cv.w};
            // lanes below nckv write the ckv row piece, the others the k row
            // (two stores, each with one descriptor for the whole wavefront)
            const int64_t ckv_off = v * ckv_row + kHalfCols * kEsz * hh + lane * 16;
            const int64_t k_off = v * kRope * 2 + (lane - nckv) * 16;
            if (lane < nckv) {
                if (buf)
                    __builtin_amdgcn_raw_buffer_store_b128(w, ckv_rsrc, (int)(uint32_t)ckv_off, 0,
                                                           kStoreSc1);
                else
                    *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(a.ckv_cache) +
                                               ckv_off) = cv;
            } else {
                if (buf)
                    __builtin_amdgcn_raw_buffer_store_b128(w, k_rsrc, (int)(uint32_t)k_off, 0,
                                                           kStoreSc1);
                else
                    *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(a.k_cache) +
                                               k_off) = cv;
            }
        }
    }
    __syncthreads();                          // the staged rows are read: LDS reused
    return kGot;
    };   // run_pass

    if (run_pass(half, 0) != kStole)
        return;
    // The partner's half, then this half again. (A loop, so that the rarely
    // used second copy of the pass is the only one besides the first.)
#pragma nounroll
    for (int pass = 1; pass <= 2; ++pass)
        run_pass(pass == 1 ? 1 - half : half, pass);

    // ---- after a takeover the pair's areas, this half's flag and its claim
    // are this workgroup's to clear (the partner resets its own claim word
    // when it starts and finds it taken) -----------------------------------
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    __hip_atomic_store(area(k, h) + 4 * lane + j, 0.0f, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
            __hip_atomic_store(flags + pair * 2 + half, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(claims + pair * 2 + half, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int64_t mla_kv_head_workspace_bytes(int64_t T)
{
    const int64_t npairs = T > 0 ? (T + kRows - 1) / kRows : 0;
    return npairs * (4 * kRows * 4 + 4 * 4);
}

// Ticks per microsecond of the current device's wall clock (the counter the
// kernel's waits read), queried once per device.
uint32_t wall_ticks_per_us()
{
    static std::atomic<uint32_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 100;
    uint32_t v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
            khz < 1000)
            khz = 100000;                     // the 100 MHz of gfx9 parts
        v = (uint32_t)(khz / 1000);
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

hipError_t launch_mla_kv_head(const MlaKvHeadArgs &a, hipStream_t stream)
{
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    const uint32_t tpu = wall_ticks_per_us();
    const uint32_t steal_ticks = a.steal_us * tpu, stall_ticks = a.stall_us * tpu;
    const int64_t npairs = (a.T + kRows - 1) / kRows;
    const int64_t grid = 16 * ((npairs + 7) / 8);   // pairs in groups of 8: b and b + 8
    const void *fn = a.ckv == 1 ? reinterpret_cast<const void *>(mla_kv_head_kernel<1>)
                   : a.ckv == 2 ? reinterpret_cast<const void *>(mla_kv_head_kernel<2>)
                                : reinterpret_cast<const void *>(mla_kv_head_kernel<0>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess)
        return e;
    if (a.ckv == 1)
        hipLaunchKernelGGL(mla_kv_head_kernel<1>, dim3((uint32_t)grid), dim3(kThreads), kLdsBytes,
                           stream, a, steal_ticks, stall_ticks);
    else if (a.ckv == 2)
        hipLaunchKernelGGL(mla_kv_head_kernel<2>, dim3((uint32_t)grid), dim3(kThreads), kLdsBytes,
                           stream, a, steal_ticks, stall_ticks);
    else
        hipLaunchKernelGGL(mla_kv_head_kernel<0>, dim3((uint32_t)grid), dim3(kThreads), kLdsBytes,
                           stream, a, steal_ticks, stall_ticks);
    return hipGetLastError();
}

}  // namespace kvrc
