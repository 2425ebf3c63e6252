/*
 * kvrc_selftest.h - numerics self-test of libkvrc's device arithmetic.
 *
 * Not part of the method. The kernels of libkvrc reach results bit-identical
 * to the float32 definition only if their building blocks round exactly as
 * IEEE float32 does; these entry points run those building blocks on the GPU
 * for caller-chosen operands so that a test can compare them with the host's
 * IEEE results and with the float8 format's definition.
 */
#ifndef KVRC_SELFTEST_H
#define KVRC_SELFTEST_H

#include <stdint.h>

#include "kvrc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * For i in [0, n), with all arrays float32 device memory of n elements
 * (16-byte aligned, outputs not overlapping inputs):
 *   q_shared[i] = the shared-divisor correctly rounded quotient a[i] / b[i]
 *                 used by the kernels (reciprocal RN(1/b[i]) plus two
 *                 corrections); meaningful on 2^-60 <= b <= 2^60,
 *                 2^-64 <= |a| <= 2^66
 *   q_ieee[i]   = a[i] / b[i] with the device's IEEE division
 *   root[i]     = sqrtf(a[i]) with the device's correctly rounded square root
 * Returns KVRC_OK, KVRC_ERR_NULL, KVRC_ERR_SHAPE (n < 0), KVRC_ERR_ALIGN,
 * KVRC_ERR_ALIAS or KVRC_ERR_HIP. Asynchronous on `stream`.
 */
int32_t kvrc_selftest_arith(const float *a, const float *b, float *q_shared, float *q_ieee,
                            float *root, int64_t n, hipStream_t stream);

/*
 * For i in [0, n): recip[i] = the reciprocal routine of the kernels applied to
 * b[i]: the hardware reciprocal estimate corrected once by Newton-Raphson with
 * an exact residual. The kernels use it only where b is in [2^-60, 2^60],
 * where it must equal the IEEE float32 1 / b[i]. b and recip are float32
 * device memory of n elements (16-byte aligned, not overlapping). Returns
 * KVRC_OK, KVRC_ERR_NULL, KVRC_ERR_SHAPE (n < 0), KVRC_ERR_ALIGN,
 * KVRC_ERR_ALIAS or KVRC_ERR_HIP. Asynchronous on `stream`.
 */
int32_t kvrc_selftest_recip(const float *b, float *recip, int64_t n, hipStream_t stream);

/*
 * For i in [0, n): code[i] = the FLOAT8 E4M3FN code the kernels store for the
 * float32 quotient x[i] (nearest E4M3FN value, ties to the even code,
 * magnitudes beyond 448 saturating to +-448; the sign bit of the code is the
 * sign of x[i], also for a zero result). Magnitudes below 464 take the
 * hardware conversion directly, as in the kernels' common path; larger ones
 * are clamped to +-448 first, as the kernels do where a quotient can get
 * there. x is float32 device memory (16-byte
 * aligned), code uint8 device memory (4-byte aligned, not overlapping x);
 * n must be a multiple of 4. Returns KVRC_OK, KVRC_ERR_NULL, KVRC_ERR_SHAPE,
 * KVRC_ERR_ALIGN, KVRC_ERR_ALIAS or KVRC_ERR_HIP. Asynchronous on `stream`.
 */
int32_t kvrc_selftest_e4m3(const float *x, uint8_t *code, int64_t n, hipStream_t stream);

/*
 * Measurement probes (not part of the method): they give a timing harness
 * the two reference points against which the kernels are read.
 *
 * kvrc_selftest_empty - launches a kernel that does nothing, with
 * `workgroups` workgroups of `threads` threads (1 <= threads <= 1024,
 * 1 <= workgroups <= 2^31 - 1): its duration is the launch and dispatch
 * floor of a grid of that shape. Returns KVRC_OK, KVRC_ERR_SHAPE or
 * KVRC_ERR_HIP. Asynchronous on `stream`.
 *
 * kvrc_selftest_copy - copies `bytes` bytes from src to dst with 16-byte
 * loads and stores (each thread moves four 16-byte pieces, all loads issued
 * before the stores; loads non-temporal, as the kernels' streaming inputs):
 * a plain device copy, the bandwidth ceiling of a kernel that moves the same
 * bytes. src and dst are device memory, 16-byte aligned and not
 * overlapping; bytes is a multiple of 16 and at most 2^40. Returns KVRC_OK
 * (also for bytes == 0: nothing launched), KVRC_ERR_NULL, KVRC_ERR_SHAPE,
 * KVRC_ERR_ALIGN, KVRC_ERR_ALIAS or KVRC_ERR_HIP. Asynchronous on `stream`.
 */
int32_t kvrc_selftest_empty(int64_t workgroups, int32_t threads, hipStream_t stream);
int32_t kvrc_selftest_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

/*
 * kvrc_selftest_mla_kv_head_stalled - kvrc_mla_kv_head_paged (same
 * arguments, status codes and results) with the second workgroup of every
 * pair held back for stall_us microseconds (0 .. 10^7) before it claims its
 * half, so that the takeover path runs: the first workgroup, finding no
 * partials and no claim from its partner, computes both halves of the pair
 * itself. When steals is not NULL (a device int32 the caller clears, 4-byte
 * aligned), the number of halves taken over is added to it. Not part of the
 * method: it lets a test check that the takeover gives the same outputs and
 * leaves the workspace zero.
 */
int32_t kvrc_selftest_mla_kv_head_stalled(const void *x, const void *w_dkv_kr, const void *gamma,
                                          float alpha_kv, const void *cos, const void *sin,
                                          const int64_t *slot_mapping, void *k_cache,
                                          void *ckv_cache, float *ckv_scale, int64_t T,
                                          int64_t He, int64_t num_blocks, int64_t block_size,
                                          int32_t ckv_dtype, float eps, void *workspace,
                                          int64_t workspace_bytes, int32_t *err_count,
                                          int64_t stall_us, int32_t *steals, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVRC_SELFTEST_H */
