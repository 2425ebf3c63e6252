// Internal launch interface between the C-ABI entry points (kvrc_api.hip,
// which validates every argument on the host) and the kernels. Nothing here
// re-validates: callers pass checked arguments only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvrc {

// Element type of the ckv cache rows (the values of kvrc_cache_dtype).
enum CkvKind : int { kCkvBf16 = 0, kCkvInt8 = 1, kCkvFp8 = 2 };

// One fused norm-rope-cache launch. Token t = b*S + s in [0, T) reads its index
// value v from index[t], or from index[b*chunks_per_seq + s/block_size] in
// block-indexed mode, and writes cache row
//   paged mode         : v
//   Norm mode          : b * rows_per_batch + v
//   block-indexed mode : (v / block_size) * block_size + s % block_size
// when 0 <= v < limit; v == -1 skips it; any other v is counted in err.
// Unsigned 32-bit division by a divisor fixed for a launch, as a
// multiply-high (Granlund and Montgomery, "Division by invariant integers
// using multiplication", the round-up method with the add-and-shift fix-up):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//   n / d = (t + ((n - t) >> 1)) >> (l - 1),   t = mulhi(n, m),
// for every 32-bit n and every d >= 2; d = 1 is marked by shift 0.
struct UDiv {
    uint32_t magic, shift;
};

inline UDiv make_udiv(uint32_t d)
{
    if (d <= 1)
        return {0, 0};
    uint32_t l = 0;
    while ((uint64_t)1 << l < d)
        ++l;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return {(uint32_t)m, l};
}

struct NormRopeCacheArgs {
    const uint16_t *kv;       // [T, Dv + Dk] bf16
    const uint16_t *gamma;    // [Dv] bf16
    const uint16_t *cos;      // [T, Dk] bf16
    const uint16_t *sin;      // [T, Dk] bf16
    const int64_t *index;     // [T]
    uint16_t *k_cache;        // [rows, Dk] bf16
    void *ckv_cache;          // [rows, Dv] bf16, int8 or E4M3FN codes
    float *ckv_scale;         // [rows] (int8 and E4M3FN only)
    int64_t T, S, Dv, Dk;
    int64_t rows_per_batch;   // > 0: Norm mode
    int64_t chunks_per_seq;   // > 0: block-indexed mode (ceil(S / block_size))
    int64_t block_size;       // block-indexed mode only
    int64_t limit;            // exclusive bound of a valid index value
    int64_t cache_rows;       // rows of each cache (paged: limit; Norm: Bc * Sc)
    UDiv div_s, div_bs;       // division by S and by block_size (both < 2^31)
    int ckv;                  // CkvKind
    float eps;
    int32_t *err;             // nullable
};

hipError_t launch_norm_rope_cache(const NormRopeCacheArgs &a, hipStream_t stream);

// One QSAPrepare launch (see qsa_prepare in kvrc.h for the semantics).
struct QsaArgs {
    const uint16_t *raw;          // [N, L, Di]
    uint16_t *block_keys;         // [N, Bcap, Di]
    const int64_t *key_length;    // [klc]
    int64_t klc;
    const float *rope_cos;        // [N, L, Dr] or null
    const float *rope_sin;
    const uint16_t *weight;       // [Di] or null
    const uint16_t *past_raw;     // [N, kbs-1, Di]
    const float *past_rope;       // [N, 2 Dr] or null
    uint16_t *next_raw;           // [N, kbs-1, Di]
    float *next_rope;             // [N, 2 Dr] or null
    int64_t N, L, Di, Dr, Bcap, kbs;
    float eps;
    int32_t *err;
};

hipError_t launch_qsa_prepare(const QsaArgs &a, hipStream_t stream);

// One MLA kv-path head launch (see kvrc_mla_kv_head_paged in kvrc.h).
struct MlaKvHeadArgs {
    const uint16_t *x;        // [T, He] bf16
    const uint16_t *w;        // [576, He] bf16
    const uint16_t *gamma;    // [512] bf16
    const uint16_t *cos;      // [T, 64] bf16
    const uint16_t *sin;      // [T, 64] bf16
    const int64_t *slot;      // [T], or nullptr with block_index
    const int64_t *block_index; // [B * chunks] (block-indexed placement), or nullptr
    int64_t S, chunks, block_size; // sequence length and chunks per sequence (block_index)
    uint16_t *k_cache;        // [cache_rows, 64] bf16
    void *ckv_cache;          // [cache_rows, 512] bf16, int8 or E4M3FN codes
    float *ckv_scale;         // [cache_rows] (int8 / E4M3FN only), else nullptr
    int32_t ckv;              // kvrc_cache_dtype
    int64_t T, He, cache_rows;
    float alpha, eps;
    void *workspace;          // mla_kv_head_workspace_bytes(T) bytes, zero between calls
    int32_t *err;             // nullable
    uint32_t tag;             // call tag in [1, 2^30): marks this call's flags and claims
    uint32_t steal_us;        // microseconds a half waits for its partner before trying
                              // to take over the partner's half
    uint32_t stall_us;        // test only (0 otherwise): half 1 of every pair waits this
                              // long before claiming its half
    int32_t *steals;          // test only (nullable): halves taken over by their partner
};

hipError_t launch_mla_kv_head(const MlaKvHeadArgs &a, hipStream_t stream);

// K granularity of the MLA head kernel (He must be a multiple of it).
constexpr int64_t kMlaHeadK = 32;
// Token rows per workgroup pair of the MLA head kernel.
constexpr int64_t kMlaPairRows = 256;
// Workspace of one MLA head call: per pair of workgroups, their per-row
// partial square sums, per-row partial maxima (quantised ckv), two ready
// flags and two claim words.
int64_t mla_kv_head_workspace_bytes(int64_t T);

// One block-selection launch (see qsa_select_topk in kvrc.h).
struct QsaSelectArgs {
    const uint16_t *query;        // [N, H, Di] bf16
    const uint16_t *keys;         // [N, Bcap, Di] bf16
    const int64_t *key_length;    // [klc]
    int64_t klc;
    float scale;
    int64_t N, H, Di, Bcap, kbs, sel, cmp, topk, Jcap;
    int64_t chunk;                // key rows staged in LDS at a time (multiple of 16)
    float *scores;                // [N, Jcap]
    int32_t *indices;             // [N, topk]
    int32_t *err;                 // nullable
};

hipError_t launch_qsa_select(const QsaSelectArgs &a, hipStream_t stream);
int64_t qsa_select_lds_bytes(int64_t H, int64_t Di, int64_t Bcap, int64_t Jcap, int64_t chunk);
// true when (H, Di, Bcap) runs on the compile-time fast path
bool qsa_select_fast_path(int64_t H, int64_t Di, int64_t Bcap);

// Largest Di qsa_prepare accepts (bounded by the per-lane accumulators).
constexpr int64_t kQsaMaxDi = 4096;

}  // namespace kvrc
