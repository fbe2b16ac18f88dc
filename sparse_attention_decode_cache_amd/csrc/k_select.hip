// k_select.hip -- stage 3: deterministic block-domain top-k.
//
// Rank blocks by (score desc, id asc), keep the first k, return them in
// ascending id order [post 10, "QSA indexer"; "block-domain top-k（COMMON-006）
// 実装は見送り"].  Each block has the 64-bit composite key
//     (order-preserving score key << 32) | ~id,
// unique and ordered exactly like (score desc, id asc), so the top k are the
// k largest composites: no ties are left to break and the chosen set is a
// function of the scores alone.
//
// Input from the score pass: every block's key, and each tile's T largest
// composites sorted descending (a tile = R consecutive blocks, T = R/8).
// One workgroup of 1024 threads, thread t owning tile t's list (registers):
//   1. a lower bound L of the k-th composite: the k-th largest TILE MAXIMUM
//      (the maxima are a subset of all blocks), one radix-refined item per
//      thread -- a few LDS passes;
//   2. the listed composites >= L (a few times k of them) go to an LDS
//      candidate list, and radix refinement marks their k largest in an LDS
//      bitmap of all N ids; kappa = the smallest marked;
//   3. exactness: a tile can hide a block >= kappa only if its list is full
//      and its last (smallest) entry is >= kappa.  If no tile is in that
//      state the marked set IS the top k; otherwise -- massive ties,
//      adversarial order -- the refinement is redone over every key;
//   4. the bitmap becomes the ascending id list by a popcount prefix sum.
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

constexpr int kT = 1024;                       // threads = tiles handled in registers
constexpr int kCand = 4096;                    // LDS candidate list
constexpr int kScanBins = 4096;
constexpr size_t kSelectMaxLds = 144 * 1024;   // of the 160 KB LDS of a gfx950 CU

struct Smem {
    uint32_t hist[kScanBins];
    uint32_t wsum[kT / 64], woff[kT / 64];
    uint64_t wmin[kT / 64], wmax[kT / 64];
    uint64_t bmin, bmax;
    uint32_t wtot, cnt, bin, above;
};

__device__ inline uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t min64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Block-wide exclusive prefix sum (ascending thread order) of one value per
// thread: DPP scan inside each wave; wave 0 scans the 16 wave totals (DPP,
// one 16-lane row) and publishes the exclusive offsets.
__device__ inline uint32_t block_excl_scan(uint32_t v, Smem &sm, uint32_t *total)
{
    const int t = threadIdx.x, w = t >> 6;
    const uint32_t x = wave::incl_scan_add(v);
    if ((t & 63) == 63)
        sm.wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        const uint32_t s = t < kT / 64 ? sm.wsum[t] : 0u;
        const uint32_t inc = wave::incl_scan_add(s);
        if (t < kT / 64)
            sm.woff[t] = inc - s;
        if (t == kT / 64 - 1)
            sm.wtot = inc;
    }
    __syncthreads();
    if (total)
        *total = sm.wtot;
    return sm.woff[w] + x - v;
}

// Block-wide min / max of one 64-bit value per thread (DPP within waves, then
// wave 0 over the 16 wave results).
__device__ inline void block_minmax(Smem &sm, uint64_t lo, uint64_t hi, uint64_t &mn, uint64_t &mx)
{
    lo = wave::reduce_min_u64(lo);
    hi = wave::reduce_max_u64(hi);
    const int t = threadIdx.x, w = t >> 6;
    if ((t & 63) == 0) {
        sm.wmin[w] = lo;
        sm.wmax[w] = hi;
    }
    __syncthreads();
    if (w == 0) {
        const uint64_t a = wave::reduce_min_u64(t < kT / 64 ? sm.wmin[t] : ~0ull);
        const uint64_t b = wave::reduce_max_u64(t < kT / 64 ? sm.wmax[t] : 0ull);
        if (t == 0) {
            sm.bmin = a;
            sm.bmax = b;
        }
    }
    __syncthreads();
    mn = sm.bmin;
    mx = sm.bmax;
    __syncthreads();
}

// Thread t owns bins [t*bpt, t*bpt + bpt) of sm.hist (ascending).  Finds the
// bin b holding the `need`-th largest item, above(b) < need <= above(b) +
// hist[b] with above(b) = items in higher bins; result in sm.bin / sm.above.
__device__ inline void find_bin(Smem &sm, int nbins, uint32_t need)
{
    const int t = threadIdx.x;
    const int bpt = (nbins + kT - 1) / kT;
    const int b0 = t * bpt;
    uint32_t mine = 0;
    for (int i = 0; i < bpt; ++i)
        if (b0 + i < nbins)
            mine += sm.hist[b0 + i];
    uint32_t total;
    const uint32_t below = block_excl_scan(mine, sm, &total);
    uint32_t acc = total - below - mine;             // items in bins above mine
    if (acc < need && acc + mine >= need) {
        for (int i = bpt - 1; i >= 0; --i) {
            const uint32_t h = b0 + i < nbins ? sm.hist[b0 + i] : 0u;
            if (acc + h >= need) {
                sm.bin = (uint32_t)(b0 + i);
                sm.above = acc;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
}

// Radix refinement over the nonzero composites visited by for_each(f): marks
// exactly `need` of them -- the largest -- via mark(comp).  The digits start
// below the leading bits shared by the smallest and the largest item, so the
// first 12-bit digit spreads the items over the histogram.
template <class ForEach, class Mark>
__device__ void refine_and_mark(Smem &sm, ForEach for_each, Mark mark, uint32_t need,
                                uint64_t *kth)
{
    uint64_t lo = ~0ull, hi = 0, mn, mx;
    for_each([&](uint64_t c) {
        lo = min64(lo, c);
        hi = max64(hi, c);
    });
    block_minmax(sm, lo, hi, mn, mx);
    if (mn == mx) {                      // a single distinct item
        for_each([&](uint64_t c) {
            if (c == mx)
                mark(c);
        });
        if (kth)
            *kth = mx;
        __syncthreads();
        return;
    }
    const int common = __clzll((long long)(mn ^ mx));
    uint64_t pmask = common == 0 ? 0ull : ~0ull << (64 - common);
    uint64_t prefix = mx & pmask;
    int width = 64 - common < 12 ? 64 - common : 12;
    int shift = 64 - common - width;
    for (;;) {
        const uint64_t dmask = (1ull << width) - 1;
        const int nbins = 1 << width;
        for (int i = threadIdx.x; i < nbins; i += kT)
            sm.hist[i] = 0u;
        __syncthreads();
        for_each([&](uint64_t c) {
            if ((c & pmask) == prefix)
                atomicAdd(&sm.hist[(c >> shift) & dmask], 1u);
        });
        __syncthreads();
        find_bin(sm, nbins, need);
        const uint32_t d = sm.bin, above = sm.above, in_d = sm.hist[d];
        for_each([&](uint64_t c) {
            if ((c & pmask) == prefix && ((c >> shift) & dmask) > d)
                mark(c);
        });
        need -= above;
        prefix |= (uint64_t)d << shift;
        pmask |= dmask << shift;
        if (in_d == need || shift == 0) {
            // Composites are unique: at shift 0 exactly one is left.  The
            // k-th largest is the smallest item under the final prefix.
            uint64_t lo2 = ~0ull;
            for_each([&](uint64_t c) {
                if ((c & pmask) == prefix) {
                    mark(c);
                    lo2 = min64(lo2, c);
                }
            });
            if (kth) {
                uint64_t a2, b2;
                block_minmax(sm, lo2, 0ull, a2, b2);
                *kth = a2;
            }
            __syncthreads();
            return;
        }
        width = shift < 8 ? shift : 8;
        shift -= width;
        __syncthreads();
    }
}

template <int kMaxT>
__global__ __launch_bounds__(kT) void k_select(SelectArgs a)
{
    extern __shared__ uint64_t dyn_lds[];
    Smem &sm = *reinterpret_cast<Smem *>(dyn_lds);
    uint64_t *cand = dyn_lds + (sizeof(Smem) + 7) / 8;
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(cand + kCand);
    const int t = threadIdx.x;
    const uint32_t nb = (uint32_t)a.nb;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t T = (uint32_t)a.T;
    const uint32_t ntiles = (uint32_t)a.ntiles;
    const uint32_t nwords = (nb + 31) >> 5;
    for (uint32_t i = t; i < nwords; i += kT)
        bitmap[i] = 0u;
    if (t == 0) {
        sm.cnt = 0;
        sm.bin = 0;
        sm.above = 0;
    }
    auto mark = [&](uint64_t c) {
        const uint32_t id = ~(uint32_t)c;
        atomicOr(&bitmap[id >> 5], 1u << (id & 31));
    };

    // This thread's tile list (sorted descending; zeros past the count).
    const bool own = (uint32_t)t < ntiles && ntiles <= (uint32_t)kT && T == (uint32_t)kMaxT;
    uint64_t lst[kMaxT];
    uint32_t cnt = 0;
    if (own) {
        cnt = a.counts[t];
        const uint4 *src = (const uint4 *)(a.lists + (size_t)t * T);
#pragma unroll
        for (int i = 0; i < kMaxT / 2; ++i) {
            if ((uint32_t)(2 * i) < T) {
                const uint4 v = src[i];
                lst[2 * i] = ((uint64_t)v.y << 32) | v.x;
                lst[2 * i + 1] = ((uint64_t)v.w << 32) | v.z;
            } else {
                lst[2 * i] = lst[2 * i + 1] = 0;
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxT; ++i)
            if ((uint32_t)i >= cnt)
                lst[i] = 0;
    } else {
#pragma unroll
        for (int i = 0; i < kMaxT; ++i)
            lst[i] = 0;
    }
    bool full = ntiles > (uint32_t)kT || T != (uint32_t)kMaxT;

    if (!full) {
        // 1. L = the k-th largest tile maximum (0 when there are <= k tiles)
        uint64_t L = 0;
        if (ntiles > k) {
            const uint64_t mx = lst[0];
            refine_and_mark(sm, [&](auto f) {
                if (mx)
                    f(mx);
            }, [&](uint64_t) {}, k, &L);
        }
        // 2. candidates: listed entries >= L
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < kMaxT; ++i)
            mine += (lst[i] != 0 && lst[i] >= L) ? 1u : 0u;
        uint32_t total;
        const uint32_t off = block_excl_scan(mine, sm, &total);
        if (total < k || total > (uint32_t)kCand) {
            full = true;
        } else {
            uint32_t o = off;
#pragma unroll
            for (int i = 0; i < kMaxT; ++i)
                if (lst[i] != 0 && lst[i] >= L)
                    cand[o++] = lst[i];
            __syncthreads();
            uint64_t kappa = 0;
            refine_and_mark(sm, [&](auto f) {
                for (uint32_t i = t; i < total; i += kT)
                    f(cand[i]);
            }, mark, k, &kappa);
            // 3. exactness check: full lists whose last entry reaches kappa
            const int bad = own && cnt == T && lst[T - 1] >= kappa ? 1 : 0;
            full = __syncthreads_or(bad) != 0;
            if (full) {
                for (uint32_t i = t; i < nwords; i += kT)
                    bitmap[i] = 0u;
                __syncthreads();
            }
        }
    }
    if (full) {
        refine_and_mark(sm, [&](auto f) {
            for (uint32_t e = t; e < nb; e += kT)
                f(comp_key(a.keys[e], e));
        }, mark, k, nullptr);
    }
    __syncthreads();

    // 4. bitmap -> ascending ids
    const uint32_t per = (nwords + kT - 1) / kT;
    const uint32_t w0 = t * per;
    const uint32_t w1 = w0 + per < nwords ? w0 + per : nwords;
    uint32_t c = 0;
    for (uint32_t w = w0; w < w1; ++w)
        c += (uint32_t)__popc(bitmap[w]);
    uint32_t o = block_excl_scan(c, sm, nullptr);
    for (uint32_t w = w0; w < w1; ++w) {
        uint32_t bits = bitmap[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            if (o < k)
                a.sel[o] = (int32_t)(w * 32 + b);
            ++o;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t s)
{
    const size_t lds = (sizeof(Smem) + 7) / 8 * 8 + 8 * (size_t)kCand + 4 * (size_t)((a.nb + 31) / 32);
    if (lds > kSelectMaxLds)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        static hipError_t attr = [] {
            hipError_t e = hipFuncSetAttribute((const void *)k_select<8>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)kSelectMaxLds);
            if (e == hipSuccess)
                e = hipFuncSetAttribute((const void *)k_select<16>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSelectMaxLds);
            if (e == hipSuccess)
                e = hipFuncSetAttribute((const void *)k_select<32>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSelectMaxLds);
            return e;
        }();
        if (attr != hipSuccess)
            return attr;
    }
    switch (a.T) {
    case 8: hipLaunchKernelGGL(k_select<8>, dim3(1), dim3(kT), lds, s, a); break;
    case 16: hipLaunchKernelGGL(k_select<16>, dim3(1), dim3(kT), lds, s, a); break;
    case 32: hipLaunchKernelGGL(k_select<32>, dim3(1), dim3(kT), lds, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qsa
