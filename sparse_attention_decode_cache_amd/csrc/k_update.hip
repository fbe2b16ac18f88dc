// k_update.hip -- stage 1 as its own launch: append the new token and/or
// rebuild summary rows [b0, b0 + nblk), one workgroup per row.  Used for bulk
// (re)builds -- prefill, rebuild after invalidation -- and for appends before
// the first completed block; a single new block is pooled inside the score
// kernel instead.  [post 10, "incremental pooled-key cache（COMMON-004）"]
#include "qsa_pool.h"

namespace qsa {
namespace {

template <bool F16>
__global__ __launch_bounds__(256) void k_update(UpdateArgs a)
{
    const int t = threadIdx.x;
    if (blockIdx.x == 0) {
        if (a.clear_ptr)
            for (int i = t; i < a.clear_words; i += 256)
                a.clear_ptr[i] = 0u;
        if (a.new_idx_row)
            append_rows(a, t, 256);
    }
    if ((int)blockIdx.x < a.nblk)
        pool_row<F16>(a, (int64_t)a.b0 + blockIdx.x, t);
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t *p, int32_t words)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < words; i += gridDim.x * 256)
        p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_iota(int32_t *p, int32_t n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        p[i] = i;
}

}  // namespace

hipError_t launch_update(const UpdateArgs &a, bool f16, hipStream_t s)
{
    const int grid = a.nblk > 0 ? a.nblk : 1;
    if (f16)
        hipLaunchKernelGGL(k_update<true>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_update<false>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(uint32_t *p, int32_t words, hipStream_t s)
{
    int grid = (words + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, s, p, words);
    return hipGetLastError();
}

hipError_t launch_iota(int32_t *p, int32_t n, hipStream_t s)
{
    int grid = (n + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
    hipLaunchKernelGGL(k_iota, dim3(grid), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace qsa
