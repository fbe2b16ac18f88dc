/* Device fills of the seeded generator (see qsagen_core.h).  Grid-stride
 * loops; every index is checked against n before the store. */
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include "qsagen_core.h"

__global__ void k_normal_f16(__half *dst, uint64_t n, uint64_t stream, uint64_t e0)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = __float2half_rn(qsagen_normal(stream, e0 + i));
}

__global__ void k_normal_f32(float *dst, uint64_t n, uint64_t stream, uint64_t e0)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = qsagen_normal(stream, e0 + i);
}

__global__ void k_unit_f32(float *dst, uint64_t n, uint64_t stream, uint64_t e0, float offset)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = offset + qsagen_unit(stream, e0 + i);
}

static unsigned grid_for(uint64_t n)
{
    uint64_t g = (n + 255) / 256;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (unsigned)g;
}

extern "C" int qsagen_dev_normal_f16(void *dst, uint64_t n, uint64_t stream, uint64_t e0,
                                     hipStream_t s)
{
    if (!dst && n) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_normal_f16, dim3(grid_for(n)), dim3(256), 0, s, (__half *)dst, n,
                       stream, e0);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int qsagen_dev_normal_f32(void *dst, uint64_t n, uint64_t stream, uint64_t e0,
                                     hipStream_t s)
{
    if (!dst && n) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0, s, (float *)dst, n,
                       stream, e0);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int qsagen_dev_unit_f32(void *dst, uint64_t n, uint64_t stream, uint64_t e0,
                                   float offset, hipStream_t s)
{
    if (!dst && n) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_unit_f32, dim3(grid_for(n)), dim3(256), 0, s, (float *)dst, n,
                       stream, e0, offset);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
