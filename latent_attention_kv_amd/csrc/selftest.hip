// Device arithmetic self-test (include/kvrc_selftest.h): runs the division
// and square-root building blocks of the kernels on caller-chosen operands.
#include "kvrc_selftest.h"

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace {

__global__ __launch_bounds__(256) void arith_kernel(const float *__restrict__ a,
                                                    const float *__restrict__ b,
                                                    float *__restrict__ qs,
                                                    float *__restrict__ qi,
                                                    float *__restrict__ root, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = a[i], y = b[i];
        const float ry = 1.0f / y;
        qs[i] = kvrc::div_rn_shared(x, y, ry);
        qi[i] = x / y;
        root[i] = sqrtf(x);
    }
}

__global__ __launch_bounds__(256) void recip_kernel(const float *__restrict__ b,
                                                    float *__restrict__ r, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        r[i] = kvrc::rcp_rn(b[i]);
}

// Four quotients per thread. Magnitudes below 464 go straight to the
// conversion (as on the kernels' path where the quotient is known to stay
// below 448 * (1 + 2^-22)); larger ones are clamped first, as the kernels do
// wherever a quotient can reach 464.
__device__ __forceinline__ float selftest_e4m3_operand(float x)
{
    return fabsf(x) < 464.0f ? x : kvrc::e4m3_clamp(x);
}

__global__ __launch_bounds__(256) void e4m3_kernel(const float4 *__restrict__ x,
                                                   uint32_t *__restrict__ code, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 v = x[i];
        code[i] = kvrc::e4m3_pack4(selftest_e4m3_operand(v.x), selftest_e4m3_operand(v.y),
                                   selftest_e4m3_operand(v.z), selftest_e4m3_operand(v.w));
    }
}

__global__ void empty_kernel() {}

// Four 16-byte pieces per thread: piece k of workgroup g, thread t is
// g * 1024 + k * 256 + t, so each load and store instruction of a wavefront
// covers 1 KiB of consecutive bytes.
__global__ __launch_bounds__(256) void copy_kernel(const kvrc::u32x4 *__restrict__ src,
                                                   kvrc::u32x4 *__restrict__ dst, int64_t n16)
{
    const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
    kvrc::u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t i = base + 256 * k;
        if (i < n16)
            v[k] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t i = base + 256 * k;
        if (i < n16)
            dst[i] = v[k];
    }
}

bool overlaps(const void *p, const void *q, int64_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes;
}

}  // namespace

extern "C" int32_t kvrc_selftest_arith(const float *a, const float *b, float *q_shared,
                                       float *q_ieee, float *root, int64_t n,
                                       hipStream_t stream)
{
    if (n < 0)
        return KVRC_ERR_SHAPE;
    if (n == 0)
        return KVRC_OK;
    if (!a || !b || !q_shared || !q_ieee || !root)
        return KVRC_ERR_NULL;
    const void *all[] = {a, b, q_shared, q_ieee, root};
    for (const void *p : all)
        if (reinterpret_cast<uintptr_t>(p) % 16)
            return KVRC_ERR_ALIGN;
    const int64_t bytes = n * 4;
    const void *outs[] = {q_shared, q_ieee, root};
    for (const void *o : outs)
        for (const void *p : all)
            if (o != p && overlaps(o, p, bytes))
                return KVRC_ERR_ALIAS;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    (void)hipGetLastError();
    hipLaunchKernelGGL(arith_kernel, dim3(grid), dim3(256), 0, stream, a, b, q_shared, q_ieee,
                       root, n);
    return hipGetLastError() == hipSuccess ? KVRC_OK : KVRC_ERR_HIP;
}

extern "C" int32_t kvrc_selftest_recip(const float *b, float *recip, int64_t n, hipStream_t stream)
{
    if (n < 0)
        return KVRC_ERR_SHAPE;
    if (n == 0)
        return KVRC_OK;
    if (!b || !recip)
        return KVRC_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(b) % 16 || reinterpret_cast<uintptr_t>(recip) % 16)
        return KVRC_ERR_ALIGN;
    if (overlaps(b, recip, n * 4))
        return KVRC_ERR_ALIAS;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    (void)hipGetLastError();
    hipLaunchKernelGGL(recip_kernel, dim3(grid), dim3(256), 0, stream, b, recip, n);
    return hipGetLastError() == hipSuccess ? KVRC_OK : KVRC_ERR_HIP;
}

extern "C" int32_t kvrc_selftest_e4m3(const float *x, uint8_t *code, int64_t n, hipStream_t stream)
{
    if (n < 0 || n % 4)
        return KVRC_ERR_SHAPE;
    if (n == 0)
        return KVRC_OK;
    if (!x || !code)
        return KVRC_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(code) % 4)
        return KVRC_ERR_ALIGN;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ca = reinterpret_cast<uintptr_t>(code);
    if (ca < xa + (uintptr_t)(n * 4) && xa < ca + (uintptr_t)n)
        return KVRC_ERR_ALIAS;
    const int64_t n4 = n / 4;
    const int64_t blocks = (n4 + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    (void)hipGetLastError();
    hipLaunchKernelGGL(e4m3_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(x), reinterpret_cast<uint32_t *>(code), n4);
    return hipGetLastError() == hipSuccess ? KVRC_OK : KVRC_ERR_HIP;
}

extern "C" int32_t kvrc_selftest_empty(int64_t workgroups, int32_t threads, hipStream_t stream)
{
    if (workgroups < 1 || workgroups > (int64_t)INT32_MAX || threads < 1 || threads > 1024)
        return KVRC_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0,
                       stream);
    return hipGetLastError() == hipSuccess ? KVRC_OK : KVRC_ERR_HIP;
}

extern "C" int32_t kvrc_selftest_copy(const void *src, void *dst, int64_t bytes,
                                      hipStream_t stream)
{
    if (bytes < 0 || bytes % 16 || bytes > ((int64_t)1 << 40))
        return KVRC_ERR_SHAPE;
    if (bytes == 0)
        return KVRC_OK;
    if (!src || !dst)
        return KVRC_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return KVRC_ERR_ALIGN;
    if (overlaps(src, dst, bytes))
        return KVRC_ERR_ALIAS;
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + 1023) / 1024;          // <= 2^26
    (void)hipGetLastError();
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const kvrc::u32x4 *>(src), static_cast<kvrc::u32x4 *>(dst), n16);
    return hipGetLastError() == hipSuccess ? KVRC_OK : KVRC_ERR_HIP;
}
