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

// q8_0 (the 8-bit K/V cache type of the runtime-tuning post, section "KV
// cacheをQ8_0にしてみる"; llama.cpp's format): 32 values share the binary16
// scale amax / 127 and are stored as round(x * 127 / amax) in int8, halves
// away from zero.  The decisions are taken in binary32 with correctly
// rounded division and product (the format's own precision).  One thread per
// 32-value block: 64 B in, 32 B of codes and 2 B of scale out.
__global__ __launch_bounds__(256) void k_q8_0_quantize(const uint16_t *x, int64_t n_blocks,
                                                       int8_t *codes, uint16_t *scales)
{
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n_blocks;
         b += (int64_t)gridDim.x * 256) {
        const uint4 *src = (const uint4 *)(x + b * 32);
        uint4 w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = src[i];
        _Float16 h[32];
        __builtin_memcpy(h, w, 64);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j)
            amax = fmaxf(amax, fabsf((float)h[j]));
        const float sc = __fdiv_rn(amax, 127.0f);
        const float inv = sc != 0.0f ? __fdiv_rn(1.0f, sc) : 0.0f;
        int8_t c[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            c[j] = (int8_t)roundf(__fmul_rn((float)h[j], inv));
        uint4 o[2];
        __builtin_memcpy(o, c, 32);
        uint4 *dst = (uint4 *)(codes + b * 32);
        dst[0] = o[0];
        dst[1] = o[1];
        scales[b] = __builtin_bit_cast(uint16_t, (_Float16)sc);
    }
}

}  // namespace

hipError_t launch_q8_0_quantize(const uint16_t *x, int64_t n_blocks, int8_t *codes, uint16_t *scales,
                                hipStream_t s)
{
    int64_t grid = (n_blocks + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 16384 ? 16384 : grid);
    hipLaunchKernelGGL(k_q8_0_quantize, dim3((unsigned)grid), dim3(256), 0, s, x, n_blocks, codes,
                       scales);
    return hipGetLastError();
}

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
