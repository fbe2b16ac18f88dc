// k_select.hip -- stage 3: deterministic block-domain top-k.
//
// Rank blocks by (score desc, id asc) and keep the first k, returned in
// ascending id order [post 10, "QSA indexer"; "block-domain top-k（COMMON-006）
// 実装は見送り"].  Every block gets the 64-bit composite key
//     (order-preserving score key << 32) | ~id,
// which is unique and orders exactly like (score desc, id asc), so "top k" is
// "composite >= the k-th largest composite" with no ties left to break.
//
// Input: the 32-bit keys and a histogram of their top 12 bits, both produced
// while scoring.  One launch:
//   A. every workgroup finds, from the histogram, the bin B1 holding the k-th
//      key and the count of keys in higher bins;
//   B. grid-stride over the keys, one key per lane: keys above B1 are sure
//      winners and are written as bitmap words (one 64-bit ballot per wave,
//      no atomics); keys inside B1 are appended to a candidate list;
//   C. the last workgroup to finish (done counter) resolves the candidates
//      with further 8-bit radix digits of the composite key until exactly k
//      are chosen, ORs them into the bitmap, then turns the bitmap into the
//      ascending id list with a popcount prefix sum.
// The chosen set is a function of the keys alone; neither the candidate order
// nor the scheduling can change it.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerThread = 4;

__device__ inline uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Block-wide exclusive prefix sum of one value per thread (256 threads).
__device__ inline uint32_t block_excl_scan(uint32_t x, uint32_t *s_tmp, uint32_t *total)
{
    const int t = threadIdx.x;
    s_tmp[t] = x;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
        const uint32_t y = t >= o ? s_tmp[t - o] : 0u;
        __syncthreads();
        s_tmp[t] += y;
        __syncthreads();
    }
    const uint32_t incl = s_tmp[t];
    if (total)
        *total = s_tmp[kThreads - 1];
    __syncthreads();
    return incl - x;
}

// Block-wide exclusive suffix sum (sum over threads with a higher index).
__device__ inline uint32_t block_excl_suffix(uint32_t x, uint32_t *s_tmp)
{
    const int t = threadIdx.x;
    s_tmp[t] = x;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
        const uint32_t y = t + o < kThreads ? s_tmp[t + o] : 0u;
        __syncthreads();
        s_tmp[t] += y;
        __syncthreads();
    }
    const uint32_t incl = s_tmp[t];
    __syncthreads();
    return incl - x;
}

__device__ inline void mark(uint64_t *bitmap, uint64_t comp)
{
    const uint32_t id = ~(uint32_t)comp;
    atomicOr((unsigned long long *)&bitmap[id >> 6], 1ull << (id & 63));
}

__global__ __launch_bounds__(kThreads) void k_select(SelectArgs a)
{
    __shared__ uint32_t s_tmp[kThreads];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_b1, s_above, s_digit, s_sufx, s_last;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const uint32_t k = (uint32_t)a.k;

    // ---- A: bin of the k-th key from the 4096-bin histogram.
    {
        constexpr int per = kHistBins / kThreads;   // 16 bins per thread
        uint32_t loc[per];
        uint32_t tot = 0;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            loc[i] = a.hist[t * per + i];
            tot += loc[i];
        }
        const uint32_t above = block_excl_suffix(tot, s_tmp);
        if (above < k && above + tot >= k) {
            uint32_t acc = above;
            for (int i = per - 1; i >= 0; --i) {
                if (acc + loc[i] >= k) {
                    s_b1 = (uint32_t)(t * per + i);
                    s_above = acc;
                    break;
                }
                acc += loc[i];
            }
        }
        __syncthreads();
    }
    const uint32_t b1 = s_b1;

    // ---- B: sure winners to the bitmap, bin-B1 keys to the candidate list.
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t base = ((int64_t)blockIdx.x * 4 + wave) * 64; base < a.nb; base += stride) {
        const int64_t i = base + lane;
        const bool in = i < a.nb;
        const uint32_t key = in ? a.keys[i] : 0u;
        const uint32_t bin = key >> (32 - kHistBits);
        const uint64_t sure = __ballot(in && bin > b1);
        const bool cnd = in && bin == b1;
        const uint64_t cm = __ballot(cnd);
        if (lane == 0)
            a.bitmap[base >> 6] = sure;
        if (cm) {
            uint32_t slot = 0;
            if (lane == 0)
                slot = atomicAdd(&a.ctrl[kCtrlCandCount], (uint32_t)__popcll(cm));
            slot = __shfl(slot, 0);
            if (cnd)
                a.cand[slot + __popcll(cm & lanemask_lt(lane))] =
                    ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)i);
        }
    }

    // ---- C: the last workgroup resolves the candidates.
    __syncthreads();
    if (t == 0) {
        __threadfence();
        const uint32_t prev = atomicAdd(&a.ctrl[kCtrlSelectDone], 1u);
        s_last = prev == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();

    const uint32_t m = __hip_atomic_load(&a.ctrl[kCtrlCandCount], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    uint32_t need = k - s_above;                 // >= 1 by the choice of B1
    uint64_t prefix = (uint64_t)b1 << (64 - kHistBits);
    uint64_t pmask = ((uint64_t)kHistBins - 1) << (64 - kHistBits);
    int width = 8;
    int shift = 64 - kHistBits - width;          // next digit: bits [shift, shift + width)
    for (;;) {
        const uint64_t dmask = (1ull << width) - 1;
        s_hist[t] = 0u;
        __syncthreads();
        for (uint32_t i = t; i < m; i += kThreads) {
            const uint64_t c = a.cand[i];
            if ((c & pmask) == prefix)
                atomicAdd(&s_hist[(c >> shift) & dmask], 1u);
        }
        __syncthreads();
        const uint32_t hv = s_hist[t];           // bins >= 2^width are zero
        const uint32_t above = block_excl_suffix(hv, s_tmp);
        if (above < need && above + hv >= need) {
            s_digit = (uint32_t)t;
            s_sufx = above;
        }
        __syncthreads();
        const uint32_t d = s_digit;
        const uint32_t sx = s_sufx;
        const uint32_t in_d = s_hist[d];
        for (uint32_t i = t; i < m; i += kThreads) {
            const uint64_t c = a.cand[i];
            if ((c & pmask) == prefix && ((c >> shift) & dmask) > d)
                mark(a.bitmap, c);
        }
        need -= sx;
        prefix |= (uint64_t)d << shift;
        pmask |= dmask << shift;
        if (in_d == need || shift == 0) {
            // Every candidate left under the prefix is chosen (composites are
            // unique, so at shift 0 exactly one is left).
            for (uint32_t i = t; i < m; i += kThreads) {
                const uint64_t c = a.cand[i];
                if ((c & pmask) == prefix)
                    mark(a.bitmap, c);
            }
            break;
        }
        width = shift < 8 ? shift : 8;
        shift -= width;
        __syncthreads();
    }
    __syncthreads();
    __threadfence();

    // Bitmap -> ascending ids.  Thread t owns a contiguous run of 64-bit words.
    const int nw = (a.nb + 63) >> 6;
    const int per = (nw + kThreads - 1) / kThreads;
    const int w0 = t * per;
    const int w1 = min(nw, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w)
        cnt += (uint32_t)__popcll(__hip_atomic_load((unsigned long long *)&a.bitmap[w],
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    uint32_t off = block_excl_scan(cnt, s_tmp, nullptr);
    for (int w = w0; w < w1; ++w) {
        uint64_t bits = __hip_atomic_load((unsigned long long *)&a.bitmap[w], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        while (bits) {
            const int bpos = __ffsll((unsigned long long)bits) - 1;
            bits &= bits - 1;
            if (off < k)
                a.sel[off] = w * 64 + bpos;
            ++off;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t s)
{
    const int64_t per_wg = (int64_t)kThreads * kKeysPerThread;
    int grid = (int)((a.nb + per_wg - 1) / per_wg);
    grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
    hipLaunchKernelGGL(k_select, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qsa
