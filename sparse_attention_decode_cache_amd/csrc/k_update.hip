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

// Block scores expanded to every cell of a block (cell 4b + j gets s[b]).
__global__ __launch_bounds__(256) void k_expand_cells(const float *scores, int32_t nb, float *cells)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < 4 * nb; i += gridDim.x * 256)
        cells[i] = scores[i >> 2];
}

// The tail cells 4 nb .. 4 nb + tail - 1 after the first `at` entries.
__global__ void k_tail_cells(int32_t *cells, int32_t at, int32_t nb, int32_t tail)
{
    if ((int)threadIdx.x < tail)
        cells[at + threadIdx.x] = 4 * nb + (int)threadIdx.x;
}

}  // namespace

hipError_t launch_expand_cells(const float *scores, int32_t nb, float *cells, hipStream_t s)
{
    int grid = (4 * nb + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 2048 ? 2048 : grid);
    hipLaunchKernelGGL(k_expand_cells, dim3(grid), dim3(256), 0, s, scores, nb, cells);
    return hipGetLastError();
}

hipError_t launch_tail_cells(int32_t *cells, int32_t at, int32_t nb, int32_t tail, hipStream_t s)
{
    hipLaunchKernelGGL(k_tail_cells, dim3(1), dim3(64), 0, s, cells, at, nb, tail);
    return hipGetLastError();
}

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
