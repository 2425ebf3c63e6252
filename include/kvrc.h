/*
 * kvrc.h - C ABI of the MI355X (gfx950) library for latent-attention KV
 * preprocessing: the fused RMSNorm + interleaved RoPE + cache scatter of the
 * per-token key row, the MLA kv-path head that produces that row from the
 * hidden state, QSAPrepare block-key compression, and block selection over
 * those keys.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is caller-owned DEVICE memory of the current HIP
 *   device. The library allocates nothing and keeps no state between calls.
 *   The MLA head entry points (kvrc_mla_kv_head_paged and _paged_blk) take
 *   a caller-owned workspace, with the rules stated at their declaration;
 *   every other entry point needs no workspace and is safe to call from
 *   several host threads at once.
 * - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *   Buffers must stay valid until that work has completed. Caches are
 *   updated in place.
 * - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16_t). All tensors
 *   are dense row-major with the shapes given below, and every base pointer
 *   must be 16-byte aligned.
 * - Problems the host can see are reported synchronously, before anything is
 *   launched, by the returned status (kvrc_status); nothing is written then.
 *   Problems only the device can see (an index out of range, a key_length
 *   smaller than L, a block beyond the capacity) skip the offending token,
 *   sequence or block, never write out of bounds, and add 1 per skipped unit
 *   to *err_count when err_count is not NULL (an int32 in device memory that
 *   the caller clears).
 * - Duplicate destination indices (where the operation requires them to be
 *   unique) are not detected; the cache contents are then undefined.
 * - Arithmetic is IEEE float32: bf16 inputs are widened exactly, each
 *   operation rounds to nearest even, and outputs are rounded to bf16
 *   (nearest even) once, at the store.
 */
#ifndef KVRC_H
#define KVRC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The same opaque type HIP uses for its streams. */
typedef struct ihipStream_t *hipStream_t;

typedef enum kvrc_status {
    KVRC_OK = 0,
    KVRC_ERR_NULL = 1,   /* a required pointer is NULL                           */
    KVRC_ERR_SHAPE = 2,  /* a size is negative or violates a shape rule          */
    KVRC_ERR_DTYPE = 3,  /* cache dtype unknown, or scale pointer does not match */
    KVRC_ERR_ALIGN = 4,  /* a base pointer is not 16-byte aligned                */
    KVRC_ERR_ALIAS = 5,  /* an output overlaps an input it must not overlap      */
    KVRC_ERR_HIP = 6,    /* the HIP runtime refused the launch (e.g. no device)  */
    KVRC_ERR_WORKSPACE = 7 /* the workspace is smaller than the call needs       */
} kvrc_status;

/* Element type of the ckv cache. */
typedef enum kvrc_cache_dtype {
    KVRC_CACHE_BF16 = 0,    /* bf16 rows, no scale                               */
    KVRC_CACHE_INT8 = 1,    /* int8 codes + one float32 scale per row            */
    KVRC_CACHE_FP8_E4M3 = 2 /* FLOAT8 E4M3FN codes + one float32 scale per row   */
} kvrc_cache_dtype;

/* Static, human-readable name of a status code. Never NULL. */
const char *kvrc_status_string(int32_t status);

/* Library ABI version (major * 100 + minor). */
int32_t kvrc_version(void);

/*
 * kvrc_paged_norm_rope_cache - fused key preprocessing into PAGED caches.
 *
 * Source: aclnnKvRmsNormRopeCache (Description; Formulas (1) interleaveRope and
 * (2) rmsNorm; restrictions on index for the PA / PA_BNSD cache modes;
 * quantisation scenario 1 for an int8 or FLOAT8 E4M3FN ckv cache) with the
 * per-row scale rule RowMax(abs)/127 and round of aclnnMlaPrologV3WeightNz
 * (Dequant Scale Query Nope formula). The source gives no scale rule for the
 * float8 cache; this library reads it as the same rule with 448, the largest
 * finite E4M3FN value, in place of 127.
 *
 * For every token t = b*S + s of kv[B, 1, S, Dv+Dk]:
 *   v = slot_mapping[t]; v == -1 skips the token (nothing is written for it;
 *   its inputs may still be read);
 *   y  = rmsnorm(kv[t, 0:Dv]) = (x / sqrt(mean(x*x) + eps)) * gamma
 *   kr = interleaved RoPE of kv[t, Dv:Dv+Dk] with cos[t], sin[t]:
 *        x1 = x[0::2], x2 = x[1::2], kr = cat(x1,x2)*cos + cat(-x2,x1)*sin
 *   ckv_cache[v / block_size, v % block_size, 0, :] = bf16(y)      (BF16), or
 *        int8 codes rint(y / scale) with scale = max|y| / 127 stored to
 *        ckv_scale[v / block_size, v % block_size, 0]             (INT8), or
 *        E4M3FN codes of y / scale (nearest, ties to the even code, +-448
 *        beyond) with scale = max|y| / 448 stored likewise   (FP8_E4M3);
 *        y / scale is the correctly rounded float32 quotient, and an
 *        all-zero row stores scale 0 and codes 0; when scale is a float32
 *        subnormal the quotient can pass 127 (448): codes saturate there
 *   k_cache[v / block_size, v % block_size, 0, :] = bf16(kr)
 * The sum of squares uses a fixed order: 64 partial sums, partial l adding
 * the squares of the 8-element chunks c = l, l+64, ... in order, folded in
 * halves (p[k] += p[k + w/2], w = 64 .. 2); results are deterministic,
 * independent of the launch, and bit-identical to the float32 definition.
 *
 * Arguments (shapes as in the source; N = 1 head):
 *   kv            bf16  [B, 1, S, Dv+Dk]
 *   gamma         bf16  [Dv]
 *   cos, sin      bf16  [B, 1, S, Dk]        one full-width row per token
 *   slot_mapping  int64 [B*S]                -1 or unique in [0, num_blocks*block_size)
 *   k_cache       bf16  [num_blocks, block_size, 1, Dk]
 *   ckv_cache     bf16, int8 or E4M3FN (uint8 codes) [num_blocks, block_size, 1, Dv]
 *   ckv_scale     float32 [num_blocks, block_size, 1]; must be NULL for BF16
 *                 and non-NULL for INT8 and FP8_E4M3
 *   Dv, Dk        multiples of 8, 8 <= Dv, Dk <= 2^20 (Dk even is the
 *                 source's rule; 8 is this library's vector width, 2^20 its
 *                 bound on a row); B*S <= 2^31 - 1; every byte size the
 *                 shapes imply must stay below 2^63 (else KVRC_ERR_SHAPE)
 *   eps           added to the mean square
 *   err_count     optional device int32, see above
 * Returns KVRC_OK (also when B*S == 0: nothing is launched and the caches are
 * untouched), or an error status with nothing written. The outputs must not
 * overlap the inputs (KVRC_ERR_ALIAS).
 */
int32_t kvrc_paged_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                                   const void *sin, const int64_t *slot_mapping, void *k_cache,
                                   void *ckv_cache, float *ckv_scale, int64_t B, int64_t S,
                                   int64_t Dv, int64_t Dk, int64_t num_blocks,
                                   int64_t block_size, int32_t ckv_dtype, float eps,
                                   int32_t *err_count, hipStream_t stream);

/*
 * kvrc_paged_blk_norm_rope_cache - the same computation into paged caches
 * addressed by one index entry per block of tokens (block-indexed mode).
 *
 * Source: aclnnKvRmsNormRopeCache, restrictions on index for the PA_BLK_BNSD
 * cache mode: the index has B * ceil(S / block_size) entries, each -1 or a
 * value in [0, num_blocks * block_size) whose quotient by block_size does not
 * repeat. Entry b * ceil(S/block_size) + c covers tokens
 * s in [c * block_size, (c + 1) * block_size) of batch b and names the
 * destination block entry / block_size; token (b, s) writes offset
 * s % block_size of that block; -1 skips the whole chunk (the last chunk of a
 * sequence may be partial).
 *
 *   block_index  int64 [B * ceil(S / block_size)]
 * Caches, other arguments, status and err_count are as for
 * kvrc_paged_norm_rope_cache (an out-of-range entry skips its chunk and
 * counts once per token of the chunk).
 */
int32_t kvrc_paged_blk_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                                       const void *sin, const int64_t *block_index,
                                       void *k_cache, void *ckv_cache, float *ckv_scale,
                                       int64_t B, int64_t S, int64_t Dv, int64_t Dk,
                                       int64_t num_blocks, int64_t block_size,
                                       int32_t ckv_dtype, float eps, int32_t *err_count,
                                       hipStream_t stream);

/*
 * kvrc_norm_rope_cache - the same computation into CONTIGUOUS (Norm mode)
 * caches.
 *
 * Source: aclnnKvRmsNormRopeCache, restrictions on index for the Norm cache
 * mode: index is [B, S] with values in [-1, Sc); a value may repeat only
 * across different batches. Batch b of kv writes batch b of the caches, so
 * Bc >= B is required.
 *
 *   index      int64 [B, S]                 -1 skips; unique within a batch row
 *   k_cache    bf16  [Bc, 1, Sc, Dk]
 *   ckv_cache  bf16, int8 or E4M3FN [Bc, 1, Sc, Dv]
 *   ckv_scale  float32 [Bc, 1, Sc] (INT8 and FP8_E4M3 only, else NULL)
 * Token (b, s) with v = index[b, s] >= 0 writes row [b, 0, v] of each cache.
 * Other arguments, the returned status and err_count are as for
 * kvrc_paged_norm_rope_cache.
 */
int32_t kvrc_norm_rope_cache(const void *kv, const void *gamma, const void *cos,
                             const void *sin, const int64_t *index, void *k_cache,
                             void *ckv_cache, float *ckv_scale, int64_t B, int64_t S, int64_t Dv,
                             int64_t Dk, int64_t Bc, int64_t Sc, int32_t ckv_dtype, float eps,
                             int32_t *err_count, hipStream_t stream);

/*
 * kvrc_mla_kv_head_workspace_bytes - bytes of device workspace that
 * kvrc_mla_kv_head_paged needs for T tokens (the first phase of the pages'
 * "workspace size, then execute" convention; 4112 bytes per 256 tokens, for
 * every ckv cache type).
 * Returns -1 for T < 0 or T > 2^31 - 1, 0 for T == 0.
 */
int64_t kvrc_mla_kv_head_workspace_bytes(int64_t T);

/*
 * kvrc_mla_kv_head_paged - the kv path of the MLA prologue: projection, then
 * the normalised key into the ckv cache and the rotated key into the k cache.
 *
 * Source: aclnnMlaPrologV3WeightNz (Interface function, third and fourth
 * paths; Formula: RmsNorm formula, c^KV = alpha_kv * RmsNorm(x W^DKV),
 * k^C = Cache(c^KV), k^R = Cache(ROPE(x W^KR))); the RoPE is Formula (1)
 * interleaveRope of aclnnKvRmsNormRopeCache, the placement its PA_BNSD rule,
 * a quantised ckv cache its quantisation scenario 1 with the RowMax/127 rule
 * of the Dequant Scale Query Nope formula (448 for FLOAT8 E4M3FN).
 *
 * For every token t of x[T, He]:
 *   c  = x[t] . W^T, float32 accumulation of the exact bf16 products (c is
 *        not rounded before the norm);
 *   y  = alpha_kv * ((c[0:512] / sqrt(mean(c[0:512]^2) + eps)) * gamma)
 *   kr = interleaved RoPE of c[512:576] with cos[t], sin[t] (as in
 *        kvrc_paged_norm_rope_cache)
 *   v = slot_mapping[t]; v == -1 skips the token;
 *   ckv_cache[v / block_size, v % block_size, 0, :] = bf16(y)       (BF16), or
 *        int8 codes of y / scale with scale = max|y| / 127 (INT8), or
 *        E4M3FN codes of y / scale with scale = max|y| / 448 (FP8_E4M3),
 *        the scale stored to ckv_scale[v / block_size, v % block_size, 0]:
 *        the per-row rule of kvrc_paged_norm_rope_cache, except that
 *        max|y| is taken as RN((1 / rms) * max|c * alpha_kv * gamma|) (the
 *        maximum before the norm, scaled) and the quotient is
 *        y * RN(1 / scale) (a few roundings more: the outputs of this head
 *        are not reproducible to the last bit anyway); codes
 *        round to nearest, ties to even, and saturate at 127 (448); an
 *        all-zero row stores scale 0 and codes 0
 *   k_cache[v / block_size, v % block_size, 0, :]   = bf16(kr)
 * The projection runs on the matrix cores in an order of its own, so the
 * outputs are not bit-reproducible against another summation order; they
 * are deterministic for a given He (independent of T and of the launch).
 *
 * Arguments:
 *   x             bf16 [T, He]
 *   w_dkv_kr      bf16 [576, He]: row j < 512 is column j of W^DKV, row
 *                 512 + i is column i of W^KR (the layout of a [out, in]
 *                 linear layer whose 576 outputs are the two weights side by
 *                 side)
 *   gamma         bf16 [512]
 *   alpha_kv      the key scale factor (a float32 scalar)
 *   cos, sin      bf16 [T, 64]
 *   slot_mapping  int64 [T]    -1 or unique in [0, num_blocks*block_size)
 *   k_cache       bf16 [num_blocks, block_size, 1, 64]
 *   ckv_cache     bf16, int8 or E4M3FN (uint8 codes) [num_blocks, block_size, 1, 512]
 *   ckv_scale     float32 [num_blocks, block_size, 1]; NULL for BF16,
 *                 non-NULL for INT8 and FP8_E4M3 (else KVRC_ERR_DTYPE)
 *   ckv_dtype     a kvrc_cache_dtype
 *   He            a multiple of 32, 32 <= He <= 2^20; T <= 2^31 - 1
 *   workspace     device memory of at least
 *                 kvrc_mla_kv_head_workspace_bytes(T) bytes (workspace_bytes
 *                 gives its size), 16-byte aligned, owned by the caller. It
 *                 must be all zero when first used; every call leaves it all
 *                 zero again, so one workspace serves any number of calls in
 *                 order on a stream (HIP graph replays included). Calls that
 *                 may run at the same time need separate workspaces.
 * Concurrency: the two workgroups that share 256 token rows exchange
 * per-row partial sums through the workspace. Neither ever waits for a
 * partner that has not started: a workgroup that finds no partials and no
 * claim from its partner after a short wait (20 us) takes the partner's
 * half over and computes both halves itself (the partner, when it starts,
 * finds its half taken and leaves); only a partner that has started - and
 * is therefore running - is waited for. MLA head calls may therefore run at
 * the same time as any other work, other MLA head calls included (on other
 * streams, each with its own workspace); the outputs are the same bits
 * whichever workgroup computes them.
 * Returns KVRC_OK (also when T == 0: nothing is launched), or an error
 * status with nothing written: KVRC_ERR_WORKSPACE when workspace_bytes is
 * too small; outputs (the workspace included) must not overlap inputs or
 * each other. err_count counts slots outside [-1, num_blocks*block_size),
 * and a workspace found not zero (a flag or claim left by another call:
 * each call marks its own with a fresh tag, so such words are ignored and
 * the outputs stay valid; zero the workspace again). It would also count a
 * started partner that published nothing for about ten seconds, which the
 * GPU's forward progress rules out (those rows would be left unwritten).
 */
int32_t kvrc_mla_kv_head_paged(const void *x, const void *w_dkv_kr, const void *gamma,
                               float alpha_kv, const void *cos, const void *sin,
                               const int64_t *slot_mapping, void *k_cache, void *ckv_cache,
                               float *ckv_scale, int64_t T, int64_t He, int64_t num_blocks,
                               int64_t block_size, int32_t ckv_dtype, float eps, void *workspace,
                               int64_t workspace_bytes, int32_t *err_count, hipStream_t stream);

/*
 * kvrc_mla_kv_head_paged_blk - the same MLA head with the BLOCK-INDEXED paged
 * placement.
 *
 * Source: aclnnMlaPrologV3WeightNz (cacheIndex of shape (B, Ceil(S/BlockSize))
 * for the PA_BLK_BSND cache mode), with the placement rule of
 * aclnnKvRmsNormRopeCache's PA_BLK_BNSD mode (restrictions on index: entries
 * -1 or in [0, num_blocks*block_size), entry / block_size not repeated).
 *
 * The T = B * S tokens of x, cos and sin are batch-major (token b*S + s is
 * position s of sequence b). Entry b * ceil(S / block_size) + c of
 * block_index covers tokens s in [c * block_size, (c + 1) * block_size) of
 * sequence b (the last chunk may be partial); it names block
 * entry / block_size, token (b, s) writes offset s % block_size of that
 * block, and -1 skips the chunk.
 *
 *   block_index  int64 [B * ceil(S / block_size)]
 * Everything else - shapes, the ckv cache types and scale,
 * workspace (kvrc_mla_kv_head_workspace_bytes(B*S) bytes), status and err_count (here an out-of-range entry skips its chunk and
 * counts once per token of the chunk) - as for kvrc_mla_kv_head_paged.
 */
int32_t kvrc_mla_kv_head_paged_blk(const void *x, const void *w_dkv_kr, const void *gamma,
                                   float alpha_kv, const void *cos, const void *sin,
                                   const int64_t *block_index, void *k_cache, void *ckv_cache,
                                   float *ckv_scale, int64_t B, int64_t S, int64_t He,
                                   int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                                   float eps, void *workspace, int64_t workspace_bytes,
                                   int32_t *err_count, hipStream_t stream);

/*
 * kvrc_mla_kv_head_paged_noalloc - kvrc_mla_kv_head_paged for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, arguments,
 * results and status codes, without the workspace arguments. The workspace
 * is a static device array of the library, one per device (2 MiB, held until
 * the process ends), so T may be at most 2^17 = 131072 tokens
 * (KVRC_ERR_WORKSPACE beyond). The call allocates nothing: the array's
 * address is looked up once per device, on the first call with that device
 * current (KVRC_ERR_HIP if that fails), and each call first clears its part
 * of the array with a small kernel on `stream`. Every call on a device
 * shares that device's array: calls that overlap on one device (different
 * streams, or host threads without ordering) race and their outputs are
 * undefined; order them on one stream, or use kvrc_mla_kv_head_paged with
 * separate workspaces.
 */
int32_t kvrc_mla_kv_head_paged_noalloc(const void *x, const void *w_dkv_kr, const void *gamma,
                                       float alpha_kv, const void *cos, const void *sin,
                                       const int64_t *slot_mapping, void *k_cache,
                                       void *ckv_cache, float *ckv_scale, int64_t T, int64_t He,
                                       int64_t num_blocks, int64_t block_size, int32_t ckv_dtype,
                                       float eps, int32_t *err_count, hipStream_t stream);

/*
 * qsa_prepare - one index key per complete key block, for sparse attention.
 *
 * Source: openvino.opset17.qsa_prepare (description and Parameters list).
 * For every sequence n:
 *   K = key_length[n] (key_length[0] for all when key_length_count == 1),
 *   P = K - L past tokens (all L new tokens are valid), r = P % kbs.
 *   History token tau is past_incomplete_raw_keys[n, tau - (P - r)] when
 *   tau < P, else raw_index_keys[n, tau - P].
 *   For every block b in [P / kbs, K / kbs) (the blocks the new tokens
 *   complete):
 *     m = (float32 sum of the block's kbs rows in token order) / kbs
 *     z = (m / sqrt(mean(m*m) + eps)) * k_norm_weight   (skipped if NULL)
 *     z[Di-Dr:Di] = interleaved RoPE (as in kvrc_paged_norm_rope_cache)
 *         with the cos/sin of token b*kbs: past_incomplete_rope[n] when
 *         b*kbs < P, else rope_cos/rope_sin[n, b*kbs - P]  (skipped if NULL)
 *     block_keys[n, b, :] = bf16(z)
 *   Carry state for the next call: r' = K % kbs, t1 = K - r';
 *     next_incomplete_raw_keys[n, i] = history token t1 + i for i < r';
 *     next_incomplete_rope[n] = cos || sin of token t1 when r' > 0.
 *   Rows of block_keys below P / kbs (the past block keys) and rows >= r' of
 *   the next state are not written.
 *
 * Arguments:
 *   raw_index_keys            bf16 [N, L, Di]
 *   block_keys                bf16 [N, Bcap, Di]   in/out (past keys in place)
 *   key_length                int64 [key_length_count], count 1 or N; read on
 *                             the device only
 *   rope_cos, rope_sin        float32 [N, L, Dr]; both NULL disables rotation
 *   k_norm_weight             bf16 [Di]; NULL disables normalisation
 *   past_incomplete_raw_keys  bf16 [N, kbs-1, Di]; rows >= P % kbs unused
 *   past_incomplete_rope      float32 [N, 2*Dr] (cos || sin); NULL iff rope off
 *   next_incomplete_raw_keys  bf16 [N, kbs-1, Di] out; must not overlap any input
 *   next_incomplete_rope      float32 [N, 2*Dr] out; NULL iff rope off
 *   Di multiple of 8, <= 4096; Dr even, 2 <= Dr <= Di when rope is on;
 *   2 <= kbs <= 2^31 - 1; L <= 2^31 - 1; every byte size the shapes imply
 *   must stay below 2^63 (else KVRC_ERR_SHAPE).
 * Returns KVRC_OK (also when N*L == 0: nothing is written, including the next
 * state), or an error status with nothing written. On the device a sequence
 * with K < L, or whose blocks reach past Bcap, is skipped (err_count).
 */
int32_t qsa_prepare(const void *raw_index_keys, void *block_keys, const int64_t *key_length,
                    int64_t key_length_count, const float *rope_cos, const float *rope_sin,
                    const void *k_norm_weight, const void *past_incomplete_raw_keys,
                    const float *past_incomplete_rope, void *next_incomplete_raw_keys,
                    float *next_incomplete_rope, int64_t N, int64_t L, int64_t Di, int64_t Dr,
                    int64_t Bcap, int64_t key_block_size, float eps, int32_t *err_count,
                    hipStream_t stream);

/*
 * qsa_select_topk - block selection for sparse attention: each sequence's
 * query heads are scored against its block keys and the best selection
 * blocks are returned.
 *
 * Source: aclnnNsaCompressAttentionInfer (Description and Formulas: P_cmp =
 * Softmax(scale * query . key^T); P_slc[j] = sum over m < l'/d and n < l/d of
 * P_cmp[(l'/d) j - m - n]; the sum over the G heads that share a key head;
 * topkIndices = topk). The compressed keys are the block keys written by
 * qsa_prepare (one per complete block of key_block_size tokens).
 *
 * For every sequence n (single-token inference: one query per head, which
 * sees all complete blocks):
 *   K = key_length[n] (key_length[0] when key_length_count == 1),
 *   nb = K / key_block_size blocks, i < nb;
 *   P_cmp[h][i] = softmax over i of scale * query[n, h] . block_keys[n, i]
 *   Q[i] = sum over the H heads of P_cmp[h][i]  (the block keys have one head)
 *   scores[n, j] = sum_{m < sel_ratio} sum_{c < cmp_ratio} Q[sel_ratio * j - m - c]
 *       (terms outside [0, nb) are 0) for j < J = (nb + sel_ratio + cmp_ratio
 *       - 3) / sel_ratio + 1 (J = 0 when nb = 0); scores[n, j] = 0 for
 *       J <= j < Jcap;
 *   indices[n, :] = the topk j < J of largest score, by descending score,
 *       equal scores by ascending j; -1 after the first min(topk, J).
 * Float32 arithmetic (bf16 products accumulated on the matrix cores, the
 * device's exp2f on scores scaled by log2 e); deterministic.
 *
 * Arguments:
 *   query         bf16 [N, H, Di]        H a multiple of 16 (<= 1024)
 *   block_keys    bf16 [N, Bcap, Di]     Di a multiple of 32 (<= 4096); rows
 *                                        >= nb do not affect the results
 *                                        (they may be read, so the whole
 *                                        array must be readable; any values,
 *                                        NaN included)
 *   key_length    int64 [key_length_count], count 1 or N; read on the device
 *   scale         the score scale (e.g. 1 / sqrt(Di))
 *   sel_ratio     l'/d >= 1 (selection block / key block), cmp_ratio l/d >= 1
 *   scores        float32 [N, Jcap] out, Jcap = (Bcap + sel_ratio + cmp_ratio - 3)
 *                 / sel_ratio + 1 (0 when Bcap = 0)
 *   indices       int32 [N, topk] out
 * A NaN score is never selected: its position, after those of every other
 * block, holds -1.
 * The working set (H + 16) (2 Di + 16) + 80 H + 4 (Bcap + Jcap + 6)
 * + 12 min(Jcap + 3, 2048) bytes (q, one 16-row key tile, per-head partial
 * results, the block scores and their ranking keys) must
 * fit one workgroup's LDS (about 160 KiB), else KVRC_ERR_SHAPE. Returns KVRC_OK (also
 * when N == 0), or an error status with nothing written; outputs must not
 * overlap inputs. A sequence with K < 0 or nb > Bcap gets scores 0 and
 * indices -1 and counts once in err_count.
 */
int32_t qsa_select_topk(const void *query, const void *block_keys, const int64_t *key_length,
                        int64_t key_length_count, float scale, int64_t N, int64_t H, int64_t Di,
                        int64_t Bcap, int64_t key_block_size, int64_t sel_ratio,
                        int64_t cmp_ratio, int64_t topk, float *scores, int32_t *indices,
                        int32_t *err_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVRC_H */
