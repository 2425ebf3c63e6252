// C-ABI entry points (include/kvrc.h): host-side validation, then one launch.
//
// Every check happens on the host before any HIP call, in this order:
// sizes and dtype -> empty input (OK, no launch) -> NULL -> alignment ->
// aliasing. Only then is the kernel launched on the caller's stream.
#include "kvrc.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "kvrc_launch.hpp"
#include "kvrc_selftest.h"

namespace {

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range span(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b)
{
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// a*b with overflow / negative guard.
bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > INT64_MAX / a)
        return false;
    *out = a * b;
    return true;
}

// *out = a*b*c*d, false if a factor is negative or the product passes
// INT64_MAX (every byte span below is formed this way, never with a bare
// multiplication).
bool prod_ok(int64_t *out, int64_t a, int64_t b, int64_t c = 1, int64_t d = 1)
{
    int64_t ab, abc;
    return mul_ok(a, b, &ab) && mul_ok(ab, c, &abc) && mul_ok(abc, d, out);
}

// Largest Dv and Dk of a norm-rope-cache row (elements), and largest He of
// the MLA head: bounds of this library, far above any model's row width,
// that keep every per-row quantity far from overflow.
constexpr int64_t kMaxRowElems = (int64_t)1 << 20;

int32_t launch_status(hipError_t e) { return e == hipSuccess ? KVRC_OK : KVRC_ERR_HIP; }

// Shared body of the norm-rope-cache entry points. `rows` is the number of
// cache rows; rows_per_batch > 0 selects Norm mode, block_size > 0 the
// block-indexed mode (one index entry per block_size tokens of a sequence).
int32_t norm_rope_cache_common(const void *kv, const void *gamma, const void *cos, const void *sin,
                               const int64_t *index, void *k_cache, void *ckv_cache,
                               float *ckv_scale, int64_t B, int64_t S, int64_t Dv, int64_t Dk,
                               int64_t rows, int64_t rows_per_batch, int64_t block_size,
                               int64_t limit, int32_t ckv_dtype, float eps, int32_t *err_count,
                               hipStream_t stream)
{
    if (ckv_dtype != KVRC_CACHE_BF16 && ckv_dtype != KVRC_CACHE_INT8 &&
        ckv_dtype != KVRC_CACHE_FP8_E4M3)
        return KVRC_ERR_DTYPE;
    if (B < 0 || S < 0 || rows < 0 || limit < 0)
        return KVRC_ERR_SHAPE;
    if (Dv < 8 || Dk < 8 || Dv % 8 || Dk % 8 || Dv > kMaxRowElems || Dk > kMaxRowElems)
        return KVRC_ERR_SHAPE;
    int64_t T;
    const int64_t D = Dv + Dk;                // <= 2^21
    if (!mul_ok(B, S, &T) || T > (int64_t)INT32_MAX)
        return KVRC_ERR_SHAPE;
    if (T == 0)
        return KVRC_OK;                       // empty input: caches untouched

    if (!kv || !gamma || !cos || !sin || !index || !k_cache || !ckv_cache)
        return KVRC_ERR_NULL;
    const bool quant = ckv_dtype != KVRC_CACHE_BF16;   // one byte per element + scale
    if (quant != (ckv_scale != nullptr))
        return KVRC_ERR_DTYPE;
    if (!aligned(kv, 16) || !aligned(gamma, 16) || !aligned(cos, 16) || !aligned(sin, 16) ||
        !aligned(index, 8) || !aligned(k_cache, 16) || !aligned(ckv_cache, 16) ||
        !aligned(ckv_scale, 4) || !aligned(err_count, 4))
        return KVRC_ERR_ALIGN;

    // ceil(S / block_size) without forming S + block_size (block_size may be
    // near 2^63 when num_blocks is 0)
    const int64_t chunks = block_size > 0 ? S / block_size + (S % block_size != 0) : 0;
    int64_t index_count = T, kbytes, cbytes, sbytes = 0, kvbytes, csbytes, ibytes;
    if ((block_size > 0 && !prod_ok(&index_count, B, chunks)) ||
        !prod_ok(&kbytes, rows, Dk, 2) || !prod_ok(&cbytes, rows, Dv, quant ? 1 : 2) ||
        (quant && !prod_ok(&sbytes, rows, 4)) || !prod_ok(&kvbytes, T, D, 2) ||
        !prod_ok(&csbytes, T, Dk, 2) || !prod_ok(&ibytes, index_count, 8))
        return KVRC_ERR_SHAPE;
    const Range in[] = {span(kv, kvbytes), span(gamma, Dv * 2), span(cos, csbytes),
                        span(sin, csbytes), span(index, ibytes)};
    const Range out[] = {span(k_cache, kbytes), span(ckv_cache, cbytes), span(ckv_scale, sbytes),
                         span(err_count, err_count ? 4 : 0)};
    for (const Range &o : out) {
        for (const Range &i : in)
            if (overlap(o, i))
                return KVRC_ERR_ALIAS;
        for (const Range &o2 : out)
            if (&o2 != &o && overlap(o, o2))
                return KVRC_ERR_ALIAS;
    }

    kvrc::NormRopeCacheArgs a;
    a.kv = static_cast<const uint16_t *>(kv);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.cos = static_cast<const uint16_t *>(cos);
    a.sin = static_cast<const uint16_t *>(sin);
    a.index = index;
    a.k_cache = static_cast<uint16_t *>(k_cache);
    a.ckv_cache = ckv_cache;
    a.ckv_scale = ckv_scale;
    a.T = T;
    a.S = S;
    a.Dv = Dv;
    a.Dk = Dk;
    a.rows_per_batch = rows_per_batch;
    a.chunks_per_seq = chunks;
    a.block_size = block_size;
    a.limit = limit;
    a.cache_rows = rows;
    a.div_s = kvrc::make_udiv((uint32_t)S);                  // S <= T < 2^31
    a.div_bs = kvrc::make_udiv((uint32_t)(block_size > 0 ? block_size : 1));
    a.ckv = ckv_dtype;
    a.eps = eps;
    a.err = err_count;
    (void)hipGetLastError();                  // start from a clean error state
    return launch_status(kvrc::launch_norm_rope_cache(a, stream));
}

}  // namespace

extern "C" {

const char *kvrc_status_string(int32_t status)
{
    switch (status) {
    case KVRC_OK: return "ok";
    case KVRC_ERR_NULL: return "required pointer is NULL";
    case KVRC_ERR_SHAPE: return "invalid size or shape";
    case KVRC_ERR_DTYPE: return "invalid cache dtype or scale pointer";
    case KVRC_ERR_ALIGN: return "pointer not aligned";
    case KVRC_ERR_ALIAS: return "output overlaps another buffer";
    case KVRC_ERR_HIP: return "HIP launch failed";
    case KVRC_ERR_WORKSPACE: return "workspace smaller than required";
    default: return "unknown status";
    }
}

int32_t kvrc_version(void) { return 106; }

int32_t kvrc_paged_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                                   const void *sin, const int64_t *slot_mapping, void *k_cache,
                                   void *ckv_cache, float *ckv_scale, int64_t B, int64_t S,
                                   int64_t Dv, int64_t Dk, int64_t num_blocks,
                                   int64_t block_size, int32_t ckv_dtype, float eps,
                                   int32_t *err_count, hipStream_t stream)
{
    int64_t rows;
    if (num_blocks < 0 || block_size < 1 || !mul_ok(num_blocks, block_size, &rows))
        return KVRC_ERR_SHAPE;
    return norm_rope_cache_common(kv, gamma, cos, sin, slot_mapping, k_cache, ckv_cache,
                                  ckv_scale, B, S, Dv, Dk, rows, 0, 0, rows, ckv_dtype, eps,
                                  err_count, stream);
}

int32_t kvrc_paged_blk_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                                       const void *sin, const int64_t *block_index,
                                       void *k_cache, void *ckv_cache, float *ckv_scale,
                                       int64_t B, int64_t S, int64_t Dv, int64_t Dk,
                                       int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                                       float eps, int32_t *err_count, hipStream_t stream)
{
    int64_t rows;
    if (num_blocks < 0 || block_size < 1 || block_size > INT32_MAX ||
        !mul_ok(num_blocks, block_size, &rows))
        return KVRC_ERR_SHAPE;
    return norm_rope_cache_common(kv, gamma, cos, sin, block_index, k_cache, ckv_cache,
                                  ckv_scale, B, S, Dv, Dk, rows, 0, block_size, rows, ckv_dtype,
                                  eps, err_count, stream);
}

int32_t kvrc_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                             const void *sin, const int64_t *index, void *k_cache,
                             void *ckv_cache, float *ckv_scale, int64_t B, int64_t S, int64_t Dv,
                             int64_t Dk, int64_t Bc, int64_t Sc, int32_t ckv_dtype, float eps,
                             int32_t *err_count, hipStream_t stream)
{
    int64_t rows;
    if (Bc < B || Sc < 0 || !mul_ok(Bc, Sc, &rows))
        return KVRC_ERR_SHAPE;
    // Sc == 0 with B*S > 0: every index must be -1; rows_per_batch stays > 0
    // only when there are rows to address.
    return norm_rope_cache_common(kv, gamma, cos, sin, index, k_cache, ckv_cache, ckv_scale, B,
                                  S, Dv, Dk, rows, Sc > 0 ? Sc : 1, 0, Sc, ckv_dtype, eps,
                                  err_count, stream);
}

int64_t kvrc_mla_kv_head_workspace_bytes(int64_t T)
{
    if (T < 0 || T > (int64_t)INT32_MAX)
        return -1;
    return kvrc::mla_kv_head_workspace_bytes(T);
}

namespace {

// Shared body of the two MLA head entry points: index = the slot mapping
// [T] (index_count = T, B = S = 0) or the block index
// [B * ceil(S / block_size)] (index_count entries, T = B * S).
// Zero `bytes` bytes (a multiple of 16) at p, 16 bytes per thread: a kernel
// rather than hipMemsetAsync, so that the clear also replays correctly in a
// captured HIP graph.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4 *p, int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_fill(void *p, int64_t bytes, hipStream_t stream)
{
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((uint32_t)((n16 + 255) / 256)), dim3(256), 0,
                       stream, static_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

// Static device scratch of the allocation-free MLA head entry point: the
// workspace of up to kNoAllocMaxTokens tokens (2^17 tokens: 512 pairs of
// workgroups, 4112 bytes each, 2 MiB), one copy per device, held until the
// process ends. In host code `scratch` is only a stand-in for the symbol:
// the device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kNoAllocMaxTokens = (int64_t)1 << 17;
constexpr int64_t kNoAllocScratchBytes = (kNoAllocMaxTokens / 256) * (4 * 256 * 4 + 4 * 4);
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (nullptr if HIP
// reports an error). The first call on a device looks it up, with that
// device current; two threads racing on the first call store the same value.
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

// Tag of an MLA head call, in [1, 2^30): the kernel marks the pair flags and
// claim words of the workspace with it, so that words left by another call
// never match this one's.
uint32_t next_mla_tag()
{
    static std::atomic<uint32_t> counter{0};
    return counter.fetch_add(1, std::memory_order_relaxed) % ((1u << 30) - 1) + 1;
}

// Microseconds a half waits for its partner's partials before it tries to
// take the partner's half over: far beyond the spread of start times of the
// two halves of a pair when both are placed, and short next to the kernel.
constexpr uint32_t kStealMicros = 20;

int32_t mla_common(const void *x, const void *w_dkv_kr, const void *gamma, float alpha_kv,
                   const void *cos, const void *sin, const int64_t *index, bool blk, int64_t B,
                   int64_t S, void *k_cache, void *ckv_cache, float *ckv_scale, int64_t T,
                   int64_t He, int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                   float eps, void *workspace, int64_t workspace_bytes, int32_t *err_count,
                   hipStream_t stream, uint32_t stall_us = 0, int32_t *steals = nullptr,
                   bool static_scratch = false)
{
    if (ckv_dtype != KVRC_CACHE_BF16 && ckv_dtype != KVRC_CACHE_INT8 &&
        ckv_dtype != KVRC_CACHE_FP8_E4M3)
        return KVRC_ERR_DTYPE;
    const bool quant = ckv_dtype != KVRC_CACHE_BF16;   // one byte per element + scale
    int64_t rows;
    if (T < 0 || T > (int64_t)INT32_MAX || He < kvrc::kMlaHeadK || He % kvrc::kMlaHeadK ||
        He > kMaxRowElems || num_blocks < 0 || block_size < 1 ||
        !mul_ok(num_blocks, block_size, &rows))
        return KVRC_ERR_SHAPE;
    const int64_t chunks = blk && S > 0 ? S / block_size + (S % block_size != 0) : 0;
    int64_t xbytes, wbytes, kbytes, cbytes, sbytes = 0, csbytes, ibytes, index_count = T;
    if (!prod_ok(&xbytes, T, He, 2) || !prod_ok(&wbytes, 576, He, 2) ||
        !prod_ok(&kbytes, rows, 64, 2) || !prod_ok(&cbytes, rows, 512, quant ? 1 : 2) ||
        (quant && !prod_ok(&sbytes, rows, 4)) || (blk && !prod_ok(&index_count, B, chunks)) ||
        !prod_ok(&ibytes, index_count, 8) || !prod_ok(&csbytes, T, 64, 2))
        return KVRC_ERR_SHAPE;
    if (T == 0)
        return KVRC_OK;                       // empty input: caches untouched
    const int64_t wsbytes = kvrc::mla_kv_head_workspace_bytes(T);
    if (static_scratch ? wsbytes > kNoAllocScratchBytes : workspace_bytes < wsbytes)
        return KVRC_ERR_WORKSPACE;
    if (!x || !w_dkv_kr || !gamma || !cos || !sin || !index || !k_cache || !ckv_cache ||
        (!static_scratch && !workspace))
        return KVRC_ERR_NULL;
    if (quant != (ckv_scale != nullptr))
        return KVRC_ERR_DTYPE;
    if (!aligned(x, 16) || !aligned(w_dkv_kr, 16) || !aligned(gamma, 16) || !aligned(cos, 16) ||
        !aligned(sin, 16) || !aligned(index, 8) || !aligned(k_cache, 16) ||
        !aligned(ckv_cache, 16) || !aligned(ckv_scale, 4) || !aligned(workspace, 16) ||
        !aligned(err_count, 4))
        return KVRC_ERR_ALIGN;
    const Range in[] = {span(x, xbytes), span(w_dkv_kr, wbytes), span(gamma, 1024),
                        span(cos, csbytes), span(sin, csbytes), span(index, ibytes)};
    const Range out[] = {span(k_cache, kbytes), span(ckv_cache, cbytes), span(ckv_scale, sbytes),
                         span(workspace, static_scratch ? 0 : wsbytes),
                         span(err_count, err_count ? 4 : 0)};
    for (const Range &o : out) {
        for (const Range &i : in)
            if (overlap(o, i))
                return KVRC_ERR_ALIAS;
        for (const Range &o2 : out)
            if (&o2 != &o && overlap(o, o2))
                return KVRC_ERR_ALIAS;
    }
    if (static_scratch) {
        // the library's own array (looked up once per device; no
        // allocation): a caller's buffer overlaps it only by pointing into it
        workspace = scratch_address();
        if (!workspace)
            return KVRC_ERR_HIP;
        const Range ws = span(workspace, wsbytes);
        for (const Range &r : in)
            if (overlap(ws, r))
                return KVRC_ERR_ALIAS;
        for (const Range &r : out)
            if (overlap(ws, r))
                return KVRC_ERR_ALIAS;
    }
    kvrc::MlaKvHeadArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w_dkv_kr);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.cos = static_cast<const uint16_t *>(cos);
    a.sin = static_cast<const uint16_t *>(sin);
    a.slot = blk ? nullptr : index;
    a.block_index = blk ? index : nullptr;
    a.S = blk ? S : 0;
    a.chunks = chunks;
    a.block_size = block_size;
    a.k_cache = static_cast<uint16_t *>(k_cache);
    a.ckv_cache = ckv_cache;
    a.ckv_scale = ckv_scale;
    a.ckv = ckv_dtype;
    a.T = T;
    a.He = He;
    a.cache_rows = rows;
    a.alpha = alpha_kv;
    a.eps = eps;
    a.workspace = workspace;
    a.err = err_count;
    a.tag = next_mla_tag();
    a.steal_us = kStealMicros;
    a.stall_us = stall_us;
    a.steals = steals;
    (void)hipGetLastError();
    if (static_scratch) {
        // the array keeps the last call's contents: clear this call's part
        const hipError_t e = launch_zero_fill(workspace, wsbytes, stream);
        if (e != hipSuccess)
            return KVRC_ERR_HIP;
    }
    return launch_status(kvrc::launch_mla_kv_head(a, stream));
}

}  // namespace

int32_t kvrc_mla_kv_head_paged(const void *x, const void *w_dkv_kr, const void *gamma,
                               float alpha_kv, const void *cos, const void *sin,
                               const int64_t *slot_mapping, void *k_cache, void *ckv_cache,
                               float *ckv_scale, int64_t T, int64_t He, int64_t num_blocks,
                               int64_t block_size, int32_t ckv_dtype, float eps, void *workspace,
                               int64_t workspace_bytes, int32_t *err_count, hipStream_t stream)
{
    return mla_common(x, w_dkv_kr, gamma, alpha_kv, cos, sin, slot_mapping, false, 0, 0, k_cache,
                      ckv_cache, ckv_scale, T, He, num_blocks, block_size, ckv_dtype, eps,
                      workspace, workspace_bytes, err_count, stream);
}

int32_t kvrc_mla_kv_head_paged_blk(const void *x, const void *w_dkv_kr, const void *gamma,
                                   float alpha_kv, const void *cos, const void *sin,
                                   const int64_t *block_index, void *k_cache, void *ckv_cache,
                                   float *ckv_scale, int64_t B, int64_t S, int64_t He,
                                   int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                                   float eps, void *workspace, int64_t workspace_bytes,
                                   int32_t *err_count, hipStream_t stream)
{
    int64_t T;
    if (B < 0 || S < 0 || !mul_ok(B, S, &T))
        return KVRC_ERR_SHAPE;
    return mla_common(x, w_dkv_kr, gamma, alpha_kv, cos, sin, block_index, true, B, S, k_cache,
                      ckv_cache, ckv_scale, T, He, num_blocks, block_size, ckv_dtype, eps,
                      workspace, workspace_bytes, err_count, stream);
}

int32_t kvrc_mla_kv_head_paged_noalloc(const void *x, const void *w_dkv_kr, const void *gamma,
                                       float alpha_kv, const void *cos, const void *sin,
                                       const int64_t *slot_mapping, void *k_cache,
                                       void *ckv_cache, float *ckv_scale, int64_t T, int64_t He,
                                       int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                                       float eps, int32_t *err_count, hipStream_t stream)
{
    return mla_common(x, w_dkv_kr, gamma, alpha_kv, cos, sin, slot_mapping, false, 0, 0, k_cache,
                      ckv_cache, ckv_scale, T, He, num_blocks, block_size, ckv_dtype, eps,
                      nullptr, 0, err_count, stream, 0, nullptr, true);
}

int32_t kvrc_selftest_mla_kv_head_stalled(const void *x, const void *w_dkv_kr, const void *gamma,
                                          float alpha_kv, const void *cos, const void *sin,
                                          const int64_t *slot_mapping, void *k_cache,
                                          void *ckv_cache, float *ckv_scale, int64_t T,
                                          int64_t He, int64_t num_blocks, int64_t block_size,
                                          int32_t ckv_dtype, float eps, void *workspace,
                                          int64_t workspace_bytes, int32_t *err_count,
                                          int64_t stall_us, int32_t *steals, hipStream_t stream)
{
    if (stall_us < 0 || stall_us > 10000000)
        return KVRC_ERR_SHAPE;
    if (steals && reinterpret_cast<uintptr_t>(steals) % 4)
        return KVRC_ERR_ALIGN;
    return mla_common(x, w_dkv_kr, gamma, alpha_kv, cos, sin, slot_mapping, false, 0, 0, k_cache,
                      ckv_cache, ckv_scale, T, He, num_blocks, block_size, ckv_dtype, eps,
                      workspace, workspace_bytes, err_count, stream,
                      (uint32_t)stall_us, steals);
}

int32_t qsa_select_topk(const void *query, const void *block_keys, const int64_t *key_length,
                        int64_t key_length_count, float scale, int64_t N, int64_t H, int64_t Di,
                        int64_t Bcap, int64_t key_block_size, int64_t sel_ratio,
                        int64_t cmp_ratio, int64_t topk, float *scores, int32_t *indices,
                        int32_t *err_count, hipStream_t stream)
{
    if (N < 0 || N > (int64_t)INT32_MAX || H < 16 || H % 16 || H > 1024 || Di < 32 || Di % 32 ||
        Di > 4096 || Bcap < 0 || Bcap > (1 << 24) || key_block_size < 1 || sel_ratio < 1 ||
        cmp_ratio < 1 || sel_ratio > 1024 || cmp_ratio > 1024 || topk < 0 ||
        topk > (int64_t)INT32_MAX)
        return KVRC_ERR_SHAPE;
    if (key_length_count != 1 && key_length_count != N)
        return KVRC_ERR_SHAPE;
    const int64_t jcap = Bcap > 0 ? (Bcap + sel_ratio + cmp_ratio - 3) / sel_ratio + 1 : 0;
    // key rows staged per chunk: as many 16-row tiles as fit (up to the
    // capacity), at least one
    constexpr int64_t kLdsBudget = 160 * 1024 - 256;
    const int64_t fixed = kvrc::qsa_select_lds_bytes(H, Di, Bcap, jcap, 0);
    const int64_t per_row = Di * 2 + 16 + H / 2;       // a staged key row, per-tile head results
    const int64_t fit = fixed < kLdsBudget ? (kLdsBudget - fixed) / per_row / 16 * 16 : 0;
    const int64_t want = (Bcap + 15) / 16 * 16;
    const int64_t chunk = want < fit ? want : fit;
    if (chunk < 16)
        return KVRC_ERR_SHAPE;
    int64_t qbytes, kbytes, sbytes, ibytes, klbytes;
    if (!prod_ok(&qbytes, N, H, Di, 2) || !prod_ok(&kbytes, N, Bcap, Di, 2) ||
        !prod_ok(&sbytes, N, jcap, 4) || !prod_ok(&ibytes, N, topk, 4) ||
        !prod_ok(&klbytes, key_length_count, 8))
        return KVRC_ERR_SHAPE;
    if (N == 0)
        return KVRC_OK;
    if (!query || !block_keys || !key_length || (sbytes && !scores) || (ibytes && !indices))
        return KVRC_ERR_NULL;
    if (!aligned(query, 16) || !aligned(block_keys, 16) || !aligned(key_length, 8) ||
        !aligned(scores, 4) || !aligned(indices, 4) || !aligned(err_count, 4))
        return KVRC_ERR_ALIGN;
    const Range in[] = {span(query, qbytes), span(block_keys, kbytes),
                        span(key_length, klbytes)};
    const Range out[] = {span(scores, sbytes), span(indices, ibytes),
                         span(err_count, err_count ? 4 : 0)};
    for (const Range &o : out) {
        for (const Range &i : in)
            if (overlap(o, i))
                return KVRC_ERR_ALIAS;
        for (const Range &o2 : out)
            if (&o2 != &o && overlap(o, o2))
                return KVRC_ERR_ALIAS;
    }
    kvrc::QsaSelectArgs a;
    a.query = static_cast<const uint16_t *>(query);
    a.keys = static_cast<const uint16_t *>(block_keys);
    a.key_length = key_length;
    a.klc = key_length_count;
    a.scale = scale;
    a.N = N;
    a.H = H;
    a.Di = Di;
    a.Bcap = Bcap;
    a.kbs = key_block_size;
    a.sel = sel_ratio;
    a.cmp = cmp_ratio;
    a.topk = topk;
    a.Jcap = jcap;
    a.chunk = chunk;
    a.scores = scores;
    a.indices = indices;
    a.err = err_count;
    (void)hipGetLastError();
    return launch_status(kvrc::launch_qsa_select(a, stream));
}

int32_t qsa_prepare(const void *raw_index_keys, void *block_keys, const int64_t *key_length,
                    int64_t key_length_count, const float *rope_cos, const float *rope_sin,
                    const void *k_norm_weight, const void *past_incomplete_raw_keys,
                    const float *past_incomplete_rope, void *next_incomplete_raw_keys,
                    float *next_incomplete_rope, int64_t N, int64_t L, int64_t Di, int64_t Dr,
                    int64_t Bcap, int64_t key_block_size, float eps, int32_t *err_count,
                    hipStream_t stream)
{
    const int64_t kbs = key_block_size;
    if (N < 0 || L < 0 || L > (int64_t)INT32_MAX || Bcap < 0 || kbs < 2 ||
        kbs > (int64_t)INT32_MAX)
        return KVRC_ERR_SHAPE;
    if (Di < 8 || Di % 8 || Di > kvrc::kQsaMaxDi)
        return KVRC_ERR_SHAPE;
    const bool rope = rope_cos != nullptr;
    if ((rope_sin != nullptr) != rope || (past_incomplete_rope != nullptr) != rope ||
        (next_incomplete_rope != nullptr) != rope)
        return KVRC_ERR_NULL;
    if (rope && (Dr < 2 || Dr % 2 || Dr > Di))
        return KVRC_ERR_SHAPE;
    if (N > 0 && key_length_count != 1 && key_length_count != N)
        return KVRC_ERR_SHAPE;
    const int64_t Drr = rope ? Dr : 0;
    int64_t NL, rowsN, capN, rawb, ropeb, pastb, stateb, capb, klbytes;
    if (!mul_ok(N, L, &NL) || !mul_ok(N, kbs - 1, &rowsN) || !mul_ok(N, Bcap, &capN) ||
        !prod_ok(&rawb, NL, Di, 2) || !prod_ok(&ropeb, NL, Drr, 4) ||
        !prod_ok(&pastb, rowsN, Di, 2) || !prod_ok(&stateb, N, 2 * Drr, 4) ||
        !prod_ok(&capb, capN, Di, 2) || !prod_ok(&klbytes, key_length_count, 8))
        return KVRC_ERR_SHAPE;
    const int64_t nb_max = (kbs - 1 + L) / kbs;       // both < 2^31
    int64_t grid;
    if (!mul_ok(N, nb_max + 1, &grid) || grid > (int64_t)INT32_MAX)
        return KVRC_ERR_SHAPE;
    if (NL == 0)
        return KVRC_OK;                       // nothing written, next state included

    if (!raw_index_keys || !block_keys || !key_length || !past_incomplete_raw_keys ||
        !next_incomplete_raw_keys)
        return KVRC_ERR_NULL;
    if (!aligned(raw_index_keys, 16) || !aligned(block_keys, 16) || !aligned(key_length, 8) ||
        !aligned(k_norm_weight, 16) || !aligned(past_incomplete_raw_keys, 16) ||
        !aligned(next_incomplete_raw_keys, 16) || !aligned(rope_cos, 4) ||
        !aligned(rope_sin, 4) || !aligned(past_incomplete_rope, 4) ||
        !aligned(next_incomplete_rope, 4) || !aligned(err_count, 4))
        return KVRC_ERR_ALIGN;

    const Range in[] = {span(raw_index_keys, rawb),
                        span(key_length, klbytes),
                        span(rope_cos, ropeb),
                        span(rope_sin, ropeb),
                        span(k_norm_weight, k_norm_weight ? Di * 2 : 0),
                        span(past_incomplete_raw_keys, pastb),
                        span(past_incomplete_rope, stateb)};
    const Range out[] = {span(block_keys, capb),
                         span(next_incomplete_raw_keys, pastb),
                         span(next_incomplete_rope, stateb),
                         span(err_count, err_count ? 4 : 0)};
    for (const Range &o : out) {
        for (const Range &i : in)
            if (overlap(o, i))
                return KVRC_ERR_ALIAS;
        for (const Range &o2 : out)
            if (&o2 != &o && overlap(o, o2))
                return KVRC_ERR_ALIAS;
    }

    kvrc::QsaArgs a;
    a.raw = static_cast<const uint16_t *>(raw_index_keys);
    a.block_keys = static_cast<uint16_t *>(block_keys);
    a.key_length = key_length;
    a.klc = key_length_count;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.weight = static_cast<const uint16_t *>(k_norm_weight);
    a.past_raw = static_cast<const uint16_t *>(past_incomplete_raw_keys);
    a.past_rope = past_incomplete_rope;
    a.next_raw = static_cast<uint16_t *>(next_incomplete_raw_keys);
    a.next_rope = next_incomplete_rope;
    a.N = N;
    a.L = L;
    a.Di = Di;
    a.Dr = Drr;
    a.Bcap = Bcap;
    a.kbs = kbs;
    a.eps = eps;
    a.err = err_count;
    (void)hipGetLastError();
    return launch_status(kvrc::launch_qsa_prepare(a, stream));
}

}  // extern "C"
