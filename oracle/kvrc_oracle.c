/*
 * CPU oracle for the fused KV preprocessing path and QSA block keys.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain definition that the
 * HIP library is checked against. Only the test suite, the smoke check and
 * the bench's CPU-baseline leg load it; the library never does, and the two
 * share no code (no header, helper, table or constant).
 *
 * Precision: every floating-point step is IEEE float32 with round to nearest
 * even, one rounding per operation, no fused multiply-add (build with
 * -ffp-contract=off). bf16 -> float32 is exact; float32 -> bf16 rounds to
 * nearest even once, at the store.
 *
 * Pinning: every function here is pinned by tests/test_oracle_*.py against
 * hand-worked cases (tests/golden/), closed forms evaluated in float64 or
 * complex128, invariants and brute-force reconstructions. No function is
 * "parity unpinned".
 *
 * Sources (page title, then the part of the page):
 *   aclnnKvRmsNormRopeCache        - Description; Formulas (1) interleaveRope
 *                                    and (2) rmsNorm; Constraints: shape
 *                                    variables, restrictions on index,
 *                                    quantisation scenario 1.
 *   aclnnMlaPrologV3WeightNz       - RmsNorm formula; Dequant Scale Query Nope
 *                                    formula (RowMax(abs)/127, round);
 *                                    Shape restrictions (empty B/S/T).
 *   openvino.opset17.qsa_prepare   - description and Parameters list.
 *
 * Readings where the pages leave a step open are marked READING below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ckv cache element types (the oracle's own numbering). */
enum { ORC_CKV_BF16 = 0, ORC_CKV_INT8 = 1, ORC_CKV_FP8 = 2 };

/* Oracle status codes (its own; unrelated to the library's). */
enum {
    ORC_OK = 0,
    ORC_BAD_ARG = 1,     /* size or pointer argument invalid             */
    ORC_BAD_INDEX = 2,   /* index/slot outside [-1, range)               */
    ORC_DUP_INDEX = 3,   /* an index/slot repeated where it must be unique */
    ORC_BAD_LENGTH = 4   /* QSA: key_length < L, or a block past capacity */
};

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)           /* NaN: keep it quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;                  /* ties go to even    */
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Row building blocks                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Sum of squares of v[0..n) in the canonical order.
 *
 * READING: the rmsNorm formula (aclnnKvRmsNormRopeCache, Formulas (2)) takes
 * the mean of x*x but fixes no summation order. A fixed order makes the sum a
 * function of the row alone, which the int8 codes need to be reproducible.
 * The order is pairwise summation over 64 partial sums:
 *   - the row is cut into chunks of 8 consecutive elements, chunk c holding
 *     elements [8c, 8c+8);
 *   - partial p[l] (l = 0..63) starts at +0 and adds, in increasing c over
 *     the chunks with c mod 64 == l, each element's square x*x (rounded
 *     product, then rounded sum), elements in increasing order;
 *   - the 64 partials are then folded in halves, level by level:
 *     p[k] <- p[k] + p[k + w/2] for k < w/2, with w = 64, 32, ..., 2.
 */
float orc_sumsq_canonical(const float *v, int64_t n)
{
    float p[64];
    for (int l = 0; l < 64; ++l)
        p[l] = 0.0f;
    for (int64_t c = 0; c * 8 < n; ++c) {
        int l = (int)(c % 64);
        int64_t end = c * 8 + 8 < n ? c * 8 + 8 : n;
        for (int64_t e = c * 8; e < end; ++e) {
            float sq = v[e] * v[e];
            p[l] = p[l] + sq;
        }
    }
    for (int w = 64; w > 1; w /= 2)
        for (int k = 0; k < w / 2; ++k)
            p[k] = p[k] + p[k + w / 2];
    return p[0];
}

/*
 * RMS normalisation of one float32 row, aclnnKvRmsNormRopeCache Formulas (2)
 * rmsNorm (also the RmsNorm formula of aclnnMlaPrologV3WeightNz):
 *   mean_square = sum(x*x) / n;  rms = sqrt(mean_square + eps);
 *   y = (x / rms) * w.
 * w == NULL means no weight (y = x / rms): the QSA weight is optional.
 * READING: the division is a true division x/rms (as printed), not a
 * multiplication by a reciprocal.
 */
void orc_rmsnorm_f32(const float *x, const float *w, int64_t n, float eps, float *y)
{
    float ss = orc_sumsq_canonical(x, n);
    float ms = ss / (float)n;
    float rms = sqrtf(ms + eps);
    for (int64_t i = 0; i < n; ++i) {
        float q = x[i] / rms;
        y[i] = w ? q * w[i] : q;
    }
}

/*
 * Interleaved RoPE of one row of even length d, aclnnKvRmsNormRopeCache
 * Formulas (1) interleaveRope:
 *   x1 = x[0::2], x2 = x[1::2]
 *   part1 = cat(x1, x2), part2 = cat(-x2, x1)
 *   y = part1 * cos + part2 * sin          (elementwise, cos/sin of width d)
 * Written out literally; the output is in half-split order, so a zero angle
 * de-interleaves the row rather than leaving it unchanged.
 */
void orc_rope_f32(const float *x, const float *cs, const float *sn, int64_t d, float *y)
{
    int64_t h = d / 2;
    float *part1 = (float *)malloc(sizeof(float) * (size_t)d);
    float *part2 = (float *)malloc(sizeof(float) * (size_t)d);
    for (int64_t i = 0; i < h; ++i) {
        float x1 = x[2 * i];
        float x2 = x[2 * i + 1];
        part1[i] = x1;
        part1[h + i] = x2;
        part2[i] = -x2;
        part2[h + i] = x1;
    }
    for (int64_t j = 0; j < d; ++j)
        y[j] = part1[j] * cs[j] + part2[j] * sn[j];
    free(part1);
    free(part2);
}

/*
 * Per-row dynamic int8 quantisation, aclnnMlaPrologV3WeightNz "Dequant Scale
 * Query Nope" formula: scale = RowMax(abs(y)) / 127; code = round(y / scale).
 * READINGS: the row is the float32 y before any bf16 rounding; round is
 * half-to-even (the pages write their formulas in torch notation, whose
 * round is half-to-even); an all-zero row stores scale 0 and codes 0.
 * While scale is a normal float32, |y/scale| <= 127*(1+2^-23) and the codes
 * fit int8. When RowMax/127 underflows into the subnormals the rounded scale
 * can be far below RowMax/127 and the quotient can pass 127: the codes then
 * saturate at +-127 (the row maximum maps to the largest code, the intent of
 * the rule).
 */
void orc_quant_row(const float *y, int64_t n, int8_t *code, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(y[i]);
        if (a > amax)
            amax = a;
    }
    float sc = amax / 127.0f;
    for (int64_t i = 0; i < n; ++i) {
        float r = sc == 0.0f ? 0.0f : rintf(y[i] / sc);
        code[i] = (int8_t)(r > 127.0f ? 127.0f : r < -127.0f ? -127.0f : r);
    }
    *scale = sc;
}

/*
 * FLOAT8 E4M3FN (one of the ckv cache types of aclnnKvRmsNormRopeCache,
 * quantisation scenario 1): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds the subnormals m * 2^-9; no infinities; codes
 * 0x7f / 0xff are NaN, so the largest finite magnitude is 0x7e = 1.75 * 2^8 =
 * 448.
 */
float orc_e4m3_decode(uint8_t c)
{
    int e = (c >> 3) & 0xf, m = c & 7;
    float mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf((float)(8 + m), e - 10);
    return (c & 0x80) ? -mag : mag;
}

/* The 127 finite non-negative E4M3FN values, indexed by code (increasing). */
static void e4m3_table(float t[127])
{
    for (int c = 0; c < 127; ++c)
        t[c] = orc_e4m3_decode((uint8_t)c);
}

/*
 * Code of the E4M3FN value nearest to v, ties to the even code; magnitudes
 * beyond 448 give 448 (saturation; the quantiser below never produces them).
 * The nearest value is found by bisection of the decoded table.
 */
static uint8_t e4m3_nearest(const float t[127], float v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= t[126])
        return sign | 126;
    int lo = 0, hi = 126;                     /* t[lo] <= a < t[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (t[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dl = a - t[lo], dh = t[hi] - a;
    int c = dl < dh ? lo : dh < dl ? hi : ((lo & 1) ? hi : lo);
    return sign | (uint8_t)c;
}

uint8_t orc_e4m3_encode(float v)
{
    float t[127];
    e4m3_table(t);
    return e4m3_nearest(t, v);
}

/*
 * Per-row dynamic FLOAT8 E4M3FN quantisation. READING: the pages give no
 * scale rule for the float8 caches; by analogy with RowMax(abs)/127 for int8
 * (aclnnMlaPrologV3WeightNz, Dequant Scale Query Nope formula: the row maximum
 * maps to the largest code), scale = RowMax(|y|) / 448 and code =
 * E4M3FN(y / scale) to nearest, ties to even. An all-zero row stores scale 0
 * and codes 0x00.
 */
void orc_quant_row_fp8(const float *y, int64_t n, uint8_t *code, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(y[i]);
        if (a > amax)
            amax = a;
    }
    float sc = amax / 448.0f;
    float t[127];
    e4m3_table(t);
    for (int64_t i = 0; i < n; ++i)
        code[i] = sc == 0.0f ? (uint8_t)0 : e4m3_nearest(t, y[i] / sc);
    *scale = sc;
}

/* ------------------------------------------------------------------------ */
/* Fused norm-rope-cache                                                    */
/* ------------------------------------------------------------------------ */

/*
 * One token: RMSNorm of kv[0..Dv) with gamma, RoPE of kv[Dv..Dv+Dk) with the
 * token's cos/sin row, results written to cache row `row` of each cache.
 * (aclnnKvRmsNormRopeCache, Description and Formulas (1), (2); quantisation
 * scenario 1 for an int8 ckv cache with the RowMax/127 rule above.)
 */
static void token_to_row(const uint16_t *kv, const float *g, const uint16_t *cs,
                         const uint16_t *sn, int64_t Dv, int64_t Dk, float eps,
                         int ckv_kind, int64_t row, uint16_t *k_cache, void *ckv_cache,
                         float *ckv_scale, float *xbuf, float *ybuf, float *cbuf, float *sbuf)
{
    /* left Dv columns: rmsNorm */
    for (int64_t i = 0; i < Dv; ++i)
        xbuf[i] = orc_bf16_to_f32(kv[i]);
    orc_rmsnorm_f32(xbuf, g, Dv, eps, ybuf);
    if (ckv_kind == ORC_CKV_INT8) {
        int8_t *dst = (int8_t *)ckv_cache + row * Dv;
        orc_quant_row(ybuf, Dv, dst, &ckv_scale[row]);
    } else if (ckv_kind == ORC_CKV_FP8) {
        uint8_t *dst = (uint8_t *)ckv_cache + row * Dv;
        orc_quant_row_fp8(ybuf, Dv, dst, &ckv_scale[row]);
    } else {
        uint16_t *dst = (uint16_t *)ckv_cache + row * Dv;
        for (int64_t i = 0; i < Dv; ++i)
            dst[i] = orc_f32_to_bf16(ybuf[i]);
    }
    /* right Dk columns: interleaved RoPE */
    for (int64_t i = 0; i < Dk; ++i) {
        xbuf[i] = orc_bf16_to_f32(kv[Dv + i]);
        cbuf[i] = orc_bf16_to_f32(cs[i]);
        sbuf[i] = orc_bf16_to_f32(sn[i]);
    }
    orc_rope_f32(xbuf, cbuf, sbuf, Dk, ybuf);
    for (int64_t i = 0; i < Dk; ++i)
        k_cache[row * Dk + i] = orc_f32_to_bf16(ybuf[i]);
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* All values in [-1, limit) and the non-(-1) values pairwise distinct. */
static int check_indices(const int64_t *idx, int64_t n, int64_t limit)
{
    for (int64_t i = 0; i < n; ++i)
        if (idx[i] < -1 || idx[i] >= limit)
            return ORC_BAD_INDEX;
    int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
    memcpy(tmp, idx, sizeof(int64_t) * (size_t)n);
    qsort(tmp, (size_t)n, sizeof(int64_t), cmp_i64);
    int rc = ORC_OK;
    for (int64_t i = 1; i < n; ++i)
        if (tmp[i] >= 0 && tmp[i] == tmp[i - 1])
            rc = ORC_DUP_INDEX;
    free(tmp);
    return rc;
}

static int run_tokens(const uint16_t *kv, const uint16_t *gamma, const uint16_t *cs,
                      const uint16_t *sn, const int64_t *dest_row, int64_t T, int64_t Dv,
                      int64_t Dk, float eps, int ckv_kind, uint16_t *k_cache, void *ckv_cache,
                      float *ckv_scale, int nthreads)
{
    float *g = (float *)malloc(sizeof(float) * (size_t)Dv);
    for (int64_t i = 0; i < Dv; ++i)
        g[i] = orc_bf16_to_f32(gamma[i]);
    int64_t wmax = Dv > Dk ? Dv : Dk;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
#endif
    {
        float *xbuf = (float *)malloc(sizeof(float) * (size_t)wmax);
        float *ybuf = (float *)malloc(sizeof(float) * (size_t)wmax);
        float *cbuf = (float *)malloc(sizeof(float) * (size_t)Dk);
        float *sbuf = (float *)malloc(sizeof(float) * (size_t)Dk);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t t = 0; t < T; ++t) {
            if (dest_row[t] < 0)
                continue;                       /* index -1: token skipped */
            token_to_row(kv + t * (Dv + Dk), g, cs + t * Dk, sn + t * Dk, Dv, Dk, eps,
                         ckv_kind, dest_row[t], k_cache, ckv_cache, ckv_scale, xbuf, ybuf,
                         cbuf, sbuf);
        }
        free(xbuf);
        free(ybuf);
        free(cbuf);
        free(sbuf);
    }
    free(g);
    (void)nthreads;
    return ORC_OK;
}

/*
 * Paged cache mode (PA / PA_BNSD with N = 1), aclnnKvRmsNormRopeCache,
 * restrictions on index: slot_mapping has B*S entries, each -1 (skip) or a
 * distinct value in [0, num_blocks*block_size). Token t = b*S + s goes to
 * block slot/block_size, offset slot%block_size of caches laid out
 * [num_blocks, block_size, 1, d]. Bytes of the caches not addressed by a
 * written token keep their value.
 */
int orc_paged_norm_rope_cache(const uint16_t *kv, const uint16_t *gamma, const uint16_t *cs,
                              const uint16_t *sn, const int64_t *slot_mapping,
                              uint16_t *k_cache, void *ckv_cache, float *ckv_scale,
                              int64_t B, int64_t S, int64_t Dv, int64_t Dk,
                              int64_t num_blocks, int64_t block_size, int ckv_kind, float eps,
                              int nthreads)
{
    if (B < 0 || S < 0 || Dv < 1 || Dk < 2 || (Dk & 1) || num_blocks < 0 || block_size < 1)
        return ORC_BAD_ARG;
    if (ckv_kind < 0 || ckv_kind > 2 || (ckv_kind != ORC_CKV_BF16 && !ckv_scale))
        return ORC_BAD_ARG;
    int64_t T = B * S;
    if (T == 0)
        return ORC_OK;                          /* empty input: caches untouched */
    int rc = check_indices(slot_mapping, T, num_blocks * block_size);
    if (rc)
        return rc;
    int64_t *dest = (int64_t *)malloc(sizeof(int64_t) * (size_t)T);
    for (int64_t t = 0; t < T; ++t) {
        int64_t v = slot_mapping[t];
        if (v < 0) {
            dest[t] = -1;
        } else {
            int64_t blk = v / block_size, off = v % block_size;
            dest[t] = (blk * block_size + off) * 1 + 0;   /* [blk, off, head 0] */
        }
    }
    rc = run_tokens(kv, gamma, cs, sn, dest, T, Dv, Dk, eps, ckv_kind, k_cache, ckv_cache,
                    ckv_scale, nthreads);
    free(dest);
    return rc;
}

/*
 * Norm (contiguous) cache mode, aclnnKvRmsNormRopeCache, restrictions on
 * index: index is [B, S] with values in [-1, Sc); a value may repeat only
 * across different batches. READING: batch b of kv writes batch b of the
 * caches [Bc, 1, Sc, d] (each batch has its own index namespace), so
 * Bc >= B is required.
 */
int orc_norm_rope_cache(const uint16_t *kv, const uint16_t *gamma, const uint16_t *cs,
                        const uint16_t *sn, const int64_t *index, uint16_t *k_cache,
                        void *ckv_cache, float *ckv_scale, int64_t B, int64_t S, int64_t Dv,
                        int64_t Dk, int64_t Bc, int64_t Sc, int ckv_kind, float eps,
                        int nthreads)
{
    if (B < 0 || S < 0 || Dv < 1 || Dk < 2 || (Dk & 1) || Bc < B || Sc < 0)
        return ORC_BAD_ARG;
    if (ckv_kind < 0 || ckv_kind > 2 || (ckv_kind != ORC_CKV_BF16 && !ckv_scale))
        return ORC_BAD_ARG;
    int64_t T = B * S;
    if (T == 0)
        return ORC_OK;
    for (int64_t b = 0; b < B; ++b) {
        int rc = check_indices(index + b * S, S, Sc);
        if (rc)
            return rc;
    }
    int64_t *dest = (int64_t *)malloc(sizeof(int64_t) * (size_t)T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            int64_t v = index[b * S + s];
            dest[b * S + s] = v < 0 ? -1 : (b * 1 + 0) * Sc + v;   /* [b, head 0, v] */
        }
    int rc = run_tokens(kv, gamma, cs, sn, dest, T, Dv, Dk, eps, ckv_kind, k_cache, ckv_cache,
                        ckv_scale, nthreads);
    free(dest);
    return rc;
}

/*
 * Block-indexed paged mode (PA_BLK_BNSD), aclnnKvRmsNormRopeCache, restrictions
 * on index: block_index holds B * ceil(S / block_size) entries, each -1 or a
 * value in [0, num_blocks*block_size) whose quotient value / block_size must
 * not repeat. READING: entry b*ceil(S/BS) + c covers the chunk of tokens
 * s in [c*BS, (c+1)*BS) of batch b; it names the destination block
 * value / BS (the quantity the page requires to be unique), and token (b, s)
 * goes to offset s mod BS of that block; -1 skips the whole chunk.
 */
int orc_paged_blk_norm_rope_cache(const uint16_t *kv, const uint16_t *gamma, const uint16_t *cs,
                                  const uint16_t *sn, const int64_t *block_index,
                                  uint16_t *k_cache, void *ckv_cache, float *ckv_scale,
                                  int64_t B, int64_t S, int64_t Dv, int64_t Dk,
                                  int64_t num_blocks, int64_t block_size, int ckv_kind,
                                  float eps, int nthreads)
{
    if (B < 0 || S < 0 || Dv < 1 || Dk < 2 || (Dk & 1) || num_blocks < 0 || block_size < 1)
        return ORC_BAD_ARG;
    if (ckv_kind < 0 || ckv_kind > 2 || (ckv_kind != ORC_CKV_BF16 && !ckv_scale))
        return ORC_BAD_ARG;
    int64_t T = B * S;
    if (T == 0)
        return ORC_OK;
    int64_t chunks = (S + block_size - 1) / block_size;
    int64_t n = B * chunks;
    int64_t *blocks = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        int64_t v = block_index[i];
        if (v < -1 || v >= num_blocks * block_size) {
            free(blocks);
            return ORC_BAD_INDEX;
        }
        blocks[i] = v < 0 ? -1 : v / block_size;
    }
    int rc = check_indices(blocks, n, num_blocks);          /* blocks must not repeat */
    free(blocks);
    if (rc)
        return rc;
    int64_t *dest = (int64_t *)malloc(sizeof(int64_t) * (size_t)T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            int64_t v = block_index[b * chunks + s / block_size];
            dest[b * S + s] = v < 0 ? -1 : (v / block_size) * block_size + s % block_size;
        }
    rc = run_tokens(kv, gamma, cs, sn, dest, T, Dv, Dk, eps, ckv_kind, k_cache, ckv_cache,
                    ckv_scale, nthreads);
    free(dest);
    return rc;
}

/* Building blocks exposed for the tests: one token, no cache. */
void orc_token_outputs(const uint16_t *kv, const uint16_t *gamma, const uint16_t *cs,
                       const uint16_t *sn, int64_t Dv, int64_t Dk, float eps, float *y_norm,
                       float *y_rope)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(Dv > Dk ? Dv : Dk));
    float *g = (float *)malloc(sizeof(float) * (size_t)Dv);
    float *c = (float *)malloc(sizeof(float) * (size_t)Dk);
    float *s = (float *)malloc(sizeof(float) * (size_t)Dk);
    for (int64_t i = 0; i < Dv; ++i) {
        x[i] = orc_bf16_to_f32(kv[i]);
        g[i] = orc_bf16_to_f32(gamma[i]);
    }
    orc_rmsnorm_f32(x, g, Dv, eps, y_norm);
    for (int64_t i = 0; i < Dk; ++i) {
        x[i] = orc_bf16_to_f32(kv[Dv + i]);
        c[i] = orc_bf16_to_f32(cs[i]);
        s[i] = orc_bf16_to_f32(sn[i]);
    }
    orc_rope_f32(x, c, s, Dk, y_rope);
    free(x);
    free(g);
    free(c);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* QSAPrepare block keys (openvino.opset17.qsa_prepare)                     */
/* ------------------------------------------------------------------------ */

/*
 * One block key from its kbs raw rows (rows[kbs][Di], bf16, in token order):
 *   m = (sum of the rows, float32, in token order) / kbs     READING: order
 *   z = rmsnorm(m) with w and eps when w != NULL, else m
 *   z[Di-Dr..Di) <- interleaved RoPE with (c, s) when c != NULL
 * m_out receives the mean, z_out the key before bf16 rounding.
 */
void orc_qsa_block_key(const uint16_t *rows, int64_t kbs, int64_t Di, const float *w,
                       const float *c, const float *s, int64_t Dr, float eps, float *m_out,
                       float *z_out)
{
    for (int64_t d = 0; d < Di; ++d)
        m_out[d] = 0.0f;
    for (int64_t t = 0; t < kbs; ++t)
        for (int64_t d = 0; d < Di; ++d)
            m_out[d] = m_out[d] + orc_bf16_to_f32(rows[t * Di + d]);
    for (int64_t d = 0; d < Di; ++d)
        m_out[d] = m_out[d] / (float)kbs;
    if (w)
        orc_rmsnorm_f32(m_out, w, Di, eps, z_out);
    else
        memcpy(z_out, m_out, sizeof(float) * (size_t)Di);
    if (c) {
        float *zr = (float *)malloc(sizeof(float) * (size_t)Dr);
        orc_rope_f32(z_out + (Di - Dr), c, s, Dr, zr);
        memcpy(z_out + (Di - Dr), zr, sizeof(float) * (size_t)Dr);
        free(zr);
    }
}

/*
 * For every sequence n (each step follows the op's description and
 * Parameters list):
 *   K  = key_length[n] (or key_length[0] when one value is given for all)
 *   P  = K - L           READING: all L new tokens are valid keys, so the
 *                        past holds K - L tokens.
 *   r  = P mod kbs       rows of the incomplete block carried in
 *                        past_incomplete_raw_keys[n, 0..r)
 *   The new tokens complete blocks b in [floor(P/kbs), floor(K/kbs)); only
 *   those are computed. Token tau of the history is carried row
 *   tau - (P - r) when tau < P, else new row tau - P.
 *   Block b is orc_qsa_block_key over tokens [b*kbs, (b+1)*kbs), rotated
 *   with the cos/sin of its first token b*kbs: the carried row
 *   past_incomplete_rope[n] = cos || sin when that token is in the past,
 *   else rope_cos/rope_sin[n, b*kbs - P].  READING: the trailing Dr dims are
 *   the rotated ones and the RoPE form is the interleaved one, the only RoPE
 *   the pages define.
 *   block_keys[n, b] = bf16(z). READING: the op's result is the full list of
 *   block keys at absolute block index; rows below floor(P/kbs) are
 *   past_block_index_keys and are left as they are.
 *   Carry state for the next call (READING: made explicit as outputs):
 *   r' = K mod kbs, t1 = K - r'; next_raw[n, i] = history token t1 + i for
 *   i < r'; when r' > 0 and rope is on, next_rope[n] = the cos || sin of
 *   token t1 (the carried row when t1 < P). Rows >= r' are not written.
 * L == 0 or N == 0: nothing is written.
 */
static const uint16_t *history_row(const uint16_t *raw, const uint16_t *past_raw, int64_t n,
                                   int64_t tau, int64_t P, int64_t r, int64_t L, int64_t Di,
                                   int64_t kbs)
{
    if (tau < P)
        return past_raw + (n * (kbs - 1) + (tau - (P - r))) * Di;
    return raw + (n * L + (tau - P)) * Di;
}

int orc_qsa_prepare(const uint16_t *raw, uint16_t *block_keys, const int64_t *key_length,
                    int64_t key_length_count, const float *rope_cos, const float *rope_sin,
                    const uint16_t *k_norm_weight, const uint16_t *past_raw,
                    const float *past_rope, uint16_t *next_raw, float *next_rope, int64_t N,
                    int64_t L, int64_t Di, int64_t Dr, int64_t Bcap, int64_t kbs, float eps,
                    int nthreads)
{
    int rope = rope_cos != NULL;
    if (N < 0 || L < 0 || Di < 1 || kbs < 2 || Bcap < 0)
        return ORC_BAD_ARG;
    if ((rope_cos == NULL) != (rope_sin == NULL))
        return ORC_BAD_ARG;
    if (rope && (Dr < 2 || (Dr & 1) || Dr > Di || !past_rope || !next_rope))
        return ORC_BAD_ARG;
    if (key_length_count != 1 && key_length_count != N)
        return ORC_BAD_ARG;
    if (N == 0 || L == 0)
        return ORC_OK;
    for (int64_t n = 0; n < N; ++n) {
        int64_t K = key_length[key_length_count == 1 ? 0 : n];
        if (K < L || K / kbs > Bcap)
            return ORC_BAD_LENGTH;
    }
    float *w = NULL;
    if (k_norm_weight) {
        w = (float *)malloc(sizeof(float) * (size_t)Di);
        for (int64_t d = 0; d < Di; ++d)
            w[d] = orc_bf16_to_f32(k_norm_weight[d]);
    }
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int64_t n = 0; n < N; ++n) {
        int64_t K = key_length[key_length_count == 1 ? 0 : n];
        int64_t P = K - L;
        int64_t r = P % kbs;
        uint16_t *rows = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(kbs * Di));
        float *m = (float *)malloc(sizeof(float) * (size_t)Di);
        float *z = (float *)malloc(sizeof(float) * (size_t)Di);
        for (int64_t b = P / kbs; b < K / kbs; ++b) {
            for (int64_t t = 0; t < kbs; ++t)
                memcpy(rows + t * Di, history_row(raw, past_raw, n, b * kbs + t, P, r, L, Di, kbs),
                       sizeof(uint16_t) * (size_t)Di);
            const float *c = NULL, *s = NULL;
            if (rope) {
                int64_t t0 = b * kbs;
                if (t0 < P) {
                    c = past_rope + n * 2 * Dr;
                    s = past_rope + n * 2 * Dr + Dr;
                } else {
                    c = rope_cos + (n * L + (t0 - P)) * Dr;
                    s = rope_sin + (n * L + (t0 - P)) * Dr;
                }
            }
            orc_qsa_block_key(rows, kbs, Di, w, c, s, Dr, eps, m, z);
            for (int64_t d = 0; d < Di; ++d)
                block_keys[(n * Bcap + b) * Di + d] = orc_f32_to_bf16(z[d]);
        }
        /* carry state */
        int64_t r2 = K % kbs, t1 = K - r2;
        for (int64_t i = 0; i < r2; ++i)
            memcpy(next_raw + (n * (kbs - 1) + i) * Di,
                   history_row(raw, past_raw, n, t1 + i, P, r, L, Di, kbs),
                   sizeof(uint16_t) * (size_t)Di);
        if (rope && r2 > 0) {
            for (int64_t j = 0; j < Dr; ++j) {
                if (t1 < P) {
                    next_rope[n * 2 * Dr + j] = past_rope[n * 2 * Dr + j];
                    next_rope[n * 2 * Dr + Dr + j] = past_rope[n * 2 * Dr + Dr + j];
                } else {
                    next_rope[n * 2 * Dr + j] = rope_cos[(n * L + (t1 - P)) * Dr + j];
                    next_rope[n * 2 * Dr + Dr + j] = rope_sin[(n * L + (t1 - P)) * Dr + j];
                }
            }
        }
        free(rows);
        free(m);
        free(z);
    }
    free(w);
    (void)nthreads;
    return ORC_OK;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Array forms of the format conversions, for the tests. */
void orc_e4m3_encode_array(const float *src, uint8_t *dst, int64_t n, int nthreads)
{
    float t[127];
    e4m3_table(t);
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < n; ++i)
        dst[i] = e4m3_nearest(t, src[i]);
    (void)nthreads;
}

void orc_f32_to_bf16_array(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_f32_to_bf16(src[i]);
}

void orc_bf16_to_f32_array(const uint16_t *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_bf16_to_f32(src[i]);
}
