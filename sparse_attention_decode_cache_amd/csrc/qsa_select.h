// qsa_select.h -- stage 3 as a workgroup routine: deterministic block-domain
// top-k.  Used by the stand-alone select kernel and, inside the attention
// kernel, by every attention workgroup (each keeps only its own blocks).
//
// Rank blocks by (score desc, id asc), keep the first k, in ascending id order
// [post 10, "QSA indexer"; "block-domain top-k（COMMON-006）実装は見送り"].
// Each block has the 64-bit composite key
//     (order-preserving score key << 32) | ~id,
// unique, nonzero and ordered exactly like (score desc, id asc), so the top k
// are the composites >= kappa, the k-th largest: no ties are left to break
// and the chosen set is a function of the scores alone.
//
// Input from the score pass: every block's key, and each tile's T largest
// composites sorted descending, zero-filled (a tile = R = 8T consecutive
// blocks).  Their union U has about N/8 entries.  1024 threads; thread t holds
// the 16-byte chunks t + 1024q of U in registers (coalesced, 8 entries).
// Fast path: a few branch-free VALU operations per entry, and the steps that
// need only one wave's worth of work done by wave 0 while the others wait
// (a barrier is cheaper than 16 copies of the same work):
//   1. min / max of the listed keys (finite scores required);
//   2. a 1024-bin histogram LINEAR in the score over [min, max] -- a monotone
//      map of the composite, so whole bins are ordered; wave 0 finds the bin
//      d holding the k-th largest (a handful of entries on scores spread like
//      sums of products; empty slots sit in bin 0, never resolved here);
//   3. the entries of bin d go to LDS; wave 0 ranks them by counting:
//      kappa = the k-th largest of U;
//   4. the winners (entries >= kappa) are marked in an LDS bitmap of the ids;
//      exactness: a tile can hide a block >= kappa only if its list is full
//      (last slot nonzero) and that last entry is >= kappa.  If none is, the
//      entries >= kappa ARE the top k of all N blocks;
//   5. thread t owns 64 ids of the bitmap; a popcount prefix sum (DPP in the
//      wave, wave totals in LDS) gives its first slot, and it hands its ids
//      to emit(slot, id) in ascending order.
// Anything the fast path cannot decide exactly -- fewer than k listed
// entries, non-finite or all-equal scores, a crowded bin, a tile that may
// hide winners, N > 65,536 -- runs the same histogram / rank / mark steps
// over every key (four passes), and where those cannot decide either, a
// radix refinement over every key; both mark the same bitmap, slots by a
// popcount prefix sum.
#pragma once
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {
namespace sel {

constexpr int kT = 1024;                       // threads
constexpr int kWaves = kT / kWave;
constexpr int kChunks = 4;                     // 16-byte list chunks held per thread
constexpr int kEntries = 2 * kChunks;          // list entries held per thread
constexpr int kFastWords = 2048;               // bitmap words of the fast path (ids < 65,536)
constexpr int kBins = kT;                      // linear bins of the fast path
constexpr int kCap = 256;                      // entries of bin d ranked by counting
constexpr size_t kMaxLds = 144 * 1024;         // of the 160 KB LDS of a gfx950 CU

struct Smem {
    uint32_t hist[kBins];
    uint64_t cand[kCap];
    alignas(16) uint32_t rmin[kWaves];
    alignas(16) uint32_t rmax[kWaves];
    alignas(16) uint32_t wtot[kWaves];
    uint64_t kappa;
    uint32_t d, need, in_d, ncand, bad, nkeep;
    // general path
    uint32_t wsum[kWaves], woff[kWaves];
    uint64_t wmin[kWaves], wmax[kWaves];
    uint64_t bmin, bmax;
    uint32_t gtot, bin, gabove;
};

// Dynamic LDS of run() with a key cache of nb words at lds_bytes(nb_max)
// when the total stays within `cap` (else without one).  Sets a.lkeys_off.
inline size_t lds_with_cache(SelectArgs &a, int32_t nb_max, size_t cap);

// Dynamic LDS of run(): Smem and the id bitmap (whole 16-byte words, so
// that a key cache placed after it is 16-byte aligned).
__host__ __device__ inline size_t lds_bytes(int32_t nb)
{
    const size_t nwords = (size_t)(nb + 31) / 32;
    const size_t bm = nwords > (size_t)kFastWords ? nwords : (size_t)kFastWords;
    return (sizeof(Smem) + 15) / 16 * 16 + 4 * ((bm + 3) / 4 * 4);
}

inline size_t lds_with_cache(SelectArgs &a, int32_t nb_max, size_t cap)
{
    const size_t base = lds_bytes(nb_max);
    const size_t with = base + 4 * (size_t)nb_max;
    a.lkeys_off = with <= cap ? (int32_t)base : 0;
    return with <= cap ? with : base;
}

// True when the fast path can hold the lists of N blocks in T-entry lists.
__host__ __device__ inline bool fits_fast(int32_t ntiles, int32_t T)
{
    return (int64_t)ntiles * T / 2 <= (int64_t)kT * kChunks;
}

__device__ inline uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t min64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Keys of finite scores: strictly between the keys of -inf and +inf.
constexpr uint32_t kKeyFiniteLo = 0x00800000u;
constexpr uint32_t kKeyFiniteHi = 0xFF7FFFFFu;

// ------------------------------------------------------------ general path

// Block-wide exclusive prefix sum (wave 0 scans the wave totals).
__device__ inline uint32_t block_excl_scan(uint32_t v, Smem &sm, uint32_t *total)
{
    const int t = threadIdx.x, w = t >> 6;
    const uint32_t x = wave::incl_scan_add(v);
    if ((t & 63) == 63)
        sm.wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        const uint32_t s = t < kWaves ? sm.wsum[t] : 0u;
        const uint32_t inc = wave::incl_scan_add(s);
        if (t < kWaves)
            sm.woff[t] = inc - s;
        if (t == kWaves - 1)
            sm.gtot = inc;
    }
    __syncthreads();
    if (total)
        *total = sm.gtot;
    return sm.woff[w] + x - v;
}

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
        const uint64_t a = wave::reduce_min_u64(t < kWaves ? sm.wmin[t] : ~0ull);
        const uint64_t b = wave::reduce_max_u64(t < kWaves ? sm.wmax[t] : 0ull);
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

// Thread t owns bins [t*bpt, t*bpt + bpt).  Finds the bin b holding the
// need-th largest item: above(b) < need <= above(b) + hist[b], above(b) =
// items in higher bins.  Result in sm.bin / sm.gabove.
__device__ inline void find_bin(Smem &sm, int nbins, uint32_t need)
{
    const int t = threadIdx.x;
    const int bpt = (nbins + kT - 1) / kT;
    const int b0 = t * bpt;
    uint32_t mine = 0;
    for (int i = 0; i < bpt; ++i)
        mine += b0 + i < nbins ? sm.hist[b0 + i] : 0u;
    uint32_t total;
    const uint32_t below = block_excl_scan(mine, sm, &total);
    uint32_t acc = total - below - mine;
    if (acc < need && acc + mine >= need) {
        for (int i = bpt - 1; i >= 0; --i) {
            const uint32_t h = b0 + i < nbins ? sm.hist[b0 + i] : 0u;
            if (acc + h >= need) {
                sm.bin = (uint32_t)(b0 + i);
                sm.gabove = acc;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
}

// Radix refinement over the composites visited by for_each(f): marks exactly
// `need` of them -- the largest -- via mark(c).  Digits start below the
// leading bits shared by the smallest and the largest item.
template <class ForEach, class Mark>
__device__ void refine_and_mark(Smem &sm, ForEach for_each, Mark mark, uint32_t need)
{
    uint64_t lo = ~0ull, hi = 0, mn, mx;
    for_each([&](uint64_t c) {
        lo = min64(lo, c);
        hi = max64(hi, c);
    });
    block_minmax(sm, lo, hi, mn, mx);
    if (mn == mx) {
        for_each([&](uint64_t c) {
            if (c == mx)
                mark(c);
        });
        __syncthreads();
        return;
    }
    const int common = __clzll((long long)(mn ^ mx));
    uint64_t pmask = common == 0 ? 0ull : ~0ull << (64 - common);
    uint64_t prefix = mx & pmask;
    int width = 64 - common < 10 ? 64 - common : 10;
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
        const uint32_t d = sm.bin, above = sm.gabove, in_d = sm.hist[d];
        for_each([&](uint64_t c) {
            if ((c & pmask) == prefix && ((c >> shift) & dmask) > d)
                mark(c);
        });
        need -= above;
        prefix |= (uint64_t)d << shift;
        pmask |= dmask << shift;
        if (in_d == need || shift == 0) {
            // composites are unique: at shift 0 exactly one is left
            for_each([&](uint64_t c) {
                if ((c & pmask) == prefix)
                    mark(c);
            });
            __syncthreads();
            return;
        }
        width = shift < 8 ? shift : 8;
        shift -= width;
        __syncthreads();
    }
}

// Emit the k ids marked in the bitmap, ascending (thread t owns a run of
// words; a block prefix sum of their popcounts gives its first slot).
template <class Emit>
__device__ void emit_bitmap(Smem &sm, const uint32_t *bitmap, uint32_t nwords, uint32_t k, Emit emit)
{
    const int t = threadIdx.x;
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
                emit(o, w * 32 + (uint32_t)b);
            ++o;
        }
    }
}

// The exact top-k over every key (radix refinement, bitmap, popcount slots).
// lkeys (LDS, nb words, or null): the keys are copied there first and every
// pass reads them from LDS instead of memory.  Whole workgroup calls;
// `bitmap` holds (nb + 31) / 32 words; emit as in run().
template <class Emit>
__device__ void general_path(const SelectArgs &a, Smem &sm, uint32_t *bitmap, uint32_t *lkeys,
                             Emit emit)
{
    const uint32_t nb = (uint32_t)a.nb;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t nwords = (nb + 31) >> 5;
    const int t = threadIdx.x;
    for (uint32_t i = t; i < nwords; i += kT)
        bitmap[i] = 0u;
    if (lkeys) {
        for (uint32_t base = 0; base < nb; base += kT * 4) {
            uint32_t kk[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t e = base + q * kT + t;
                kk[q] = a.keys[e < nb ? e : nb - 1];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t e = base + q * kT + t;
                if (e < nb)
                    lkeys[e] = kk[q];
            }
        }
    }
    __syncthreads();
    auto each_key = [&](auto f) {
        if (lkeys) {
            for (uint32_t e = t; e < nb; e += kT)
                f(comp_key(lkeys[e], e));
            return;
        }
        for (uint32_t base = 0; base < nb; base += kT * 8) {
            uint32_t kk[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t e = base + q * kT + t;
                kk[q] = a.keys[e < nb ? e : nb - 1];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t e = base + q * kT + t;
                if (e < nb)
                    f(comp_key(kk[q], e));
            }
        }
    };
    refine_and_mark(sm, each_key, [&](uint64_t c) {
        const uint32_t id = ~(uint32_t)c;
        atomicOr(&bitmap[id >> 5], 1u << (id & 31));
    }, k);
    __syncthreads();
    emit_bitmap(sm, bitmap, nwords, k, emit);
}

// The exact top-k over every key: min / max, a 1024-bin histogram linear in
// the score (or in the key when every score is >= 0), the entries of the bin
// holding the k-th ranked by counting (kappa = the k-th largest composite),
// the composites >= kappa marked.  A lower bound tau <= kappa prunes the
// later passes: each thread's largest key is one of the keys, so if k of
// these maxima are >= tau, at least k keys are, and the k-th largest is too.
// tau is the k-th largest maximum (found by the same histogram / rank steps
// on the 1024 maxima), and only keys >= tau -- a few per cent -- enter the
// histogram, the boundary bin and the marks.  Non-finite scores or a
// crowded bin fall back to the radix refinement.  lkeys (LDS, nb words, or
// null): the keys are read from memory once and kept there.  keep (LDS,
// keep_cap composites, or null): the histogram pass also lists the keys >=
// tau there, and the marking pass walks that list instead of every key
// when it held them all (the same keys, so the same marks).  Requires
// nb > k.  Whole workgroup calls; emit as in run().
template <class Emit>
__device__ void keys_path(const SelectArgs &a, Smem &sm, uint32_t *bitmap, uint32_t *lkeys, Emit emit,
                          uint64_t *keep = nullptr, uint32_t keep_cap = 0u)
{
    const uint32_t nb = (uint32_t)a.nb;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t nwords = (nb + 31) >> 5;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    for (uint32_t i = t; i < nwords; i += kT)
        bitmap[i] = 0u;
    sm.hist[t] = 0u;
    if (t == 0) {
        sm.ncand = 0u;
        sm.nkeep = 0u;
        sm.d = 0xFFFFFFFFu;
    }
    // 1. keys (to LDS when asked), their range, and this thread's largest;
    //    in 16-byte chunks of 4 keys (the keys are 16-byte aligned), 8 per
    //    thread in flight (32,768 keys a memory latency), the last nb % 4
    //    keys one by one (nothing past nb is read)
    const uint32_t nch = nb >> 2, ntail = nb & 3u;
    const uint4 *keys4 = reinterpret_cast<const uint4 *>(a.keys);
    constexpr int kRound = 8;
    uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;
    auto see = [&](uint32_t key) __attribute__((always_inline)) {
        kmin1 = min(kmin1, key - 1u);
        kmax = max(kmax, key);
    };
    for (uint32_t base = 0; base < nch; base += kT * kRound) {
        uint4 kk[kRound];
#pragma unroll
        for (int q = 0; q < kRound; ++q) {
            const uint32_t c = base + q * kT + t;
            kk[q] = keys4[c < nch ? c : nch - 1];
        }
#pragma unroll
        for (int q = 0; q < kRound; ++q) {
            const uint32_t c = base + q * kT + t;
            if (c < nch) {
                if (lkeys)
                    *reinterpret_cast<uint4 *>(lkeys + 4 * c) = kk[q];
                see(kk[q].x);
                see(kk[q].y);
                see(kk[q].z);
                see(kk[q].w);
            }
        }
    }
    if ((uint32_t)t < ntail) {
        const uint32_t e = 4 * nch + t, key = a.keys[e];
        if (lkeys)
            lkeys[e] = key;
        see(key);
    }
    // this thread's largest key (it holds one iff it took a chunk or a tail key)
    const uint32_t tmax = kmax;
    const bool holds = (uint32_t)t < nch || (uint32_t)t < ntail;
    kmin1 = wave::reduce_min_u32(kmin1);
    kmax = wave::reduce_max_u32(kmax);
    if (lane == 0) {
        sm.rmin[wv] = kmin1;
        sm.rmax[wv] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; i += 4) {
        const uint4 a4 = reinterpret_cast<const uint4 *>(sm.rmin)[i / 4];
        const uint4 b4 = reinterpret_cast<const uint4 *>(sm.rmax)[i / 4];
        kmin1 = min(min(kmin1, a4.x), min(a4.y, min(a4.z, a4.w)));
        kmax = max(max(kmax, b4.x), max(b4.y, max(b4.z, b4.w)));
    }
    const uint32_t kmin = kmin1 + 1u;
    const float mn = key_score(kmin), mx = key_score(kmax);
    const float range = mx - mn;
    const float scale = (float)kBins / range;
    bool general = kmin < kKeyFiniteLo || kmax > kKeyFiniteHi || !(range > 0.0f) ||
                   !(range < __builtin_inff()) || !(scale < __builtin_inff());
    const bool by_key = kmin >= 0x80000000u;
    const int kshift = 32 - __clz((int)(kmax - kmin)) - 10;
    const uint32_t ksh = kshift > 0 ? (uint32_t)kshift : 0u;
    // f(key, id) for every key, a 16-byte chunk at a time
    auto each_key = [&](auto f) __attribute__((always_inline)) {
        for (uint32_t c = t; c < nch; c += kT) {
            const uint4 v = lkeys ? *reinterpret_cast<const uint4 *>(lkeys + 4 * c) : keys4[c];
            f(v.x, 4 * c);
            f(v.y, 4 * c + 1);
            f(v.z, 4 * c + 2);
            f(v.w, 4 * c + 3);
        }
        if ((uint32_t)t < ntail) {
            const uint32_t e = 4 * nch + t;
            f(lkeys ? lkeys[e] : a.keys[e], e);
        }
    };
    auto bin_of = [&](uint32_t key) -> uint32_t {
        if (by_key)
            return (key > kmin ? key - kmin : 0u) >> ksh;
        const float sc = fmaxf(key_score(key), mn);
        const uint32_t b = (uint32_t)((sc - mn) * scale);
        return b < (uint32_t)kBins - 1 ? b : (uint32_t)kBins - 1;
    };
    // The bin holding the need-th largest of the histogram (thread t takes
    // bin 1023 - t): sm.d, sm.need (rank inside the bin), sm.in_d.
    auto kth_bin = [&](uint32_t need) {
        const uint32_t h = sm.hist[kBins - 1 - t];
        const uint32_t incl = wave::incl_scan_add(h);
        if (lane == 63)
            sm.wtot[wv] = incl;
        __syncthreads();
        uint32_t off = 0;
#pragma unroll
        for (int i = 0; i < kWaves; i += 4) {
            const uint4 w4 = reinterpret_cast<const uint4 *>(sm.wtot)[i / 4];
            off += (i < wv ? w4.x : 0u) + (i + 1 < wv ? w4.y : 0u) + (i + 2 < wv ? w4.z : 0u) +
                   (i + 3 < wv ? w4.w : 0u);
        }
        const uint32_t above = off + incl - h;
        if (above < need && above + h >= need) {
            sm.d = (uint32_t)(kBins - 1 - t);
            sm.need = need - above;
            sm.in_d = h;
        }
        __syncthreads();
    };
    // wave 0 ranks the m candidates by counting: sm.kappa = the need-th largest
    auto rank_cand = [&](uint32_t m, uint32_t need) {
        if (wv == 0) {
            for (uint32_t j = lane; j < m; j += kWave) {
                const uint64_t c = sm.cand[j];
                uint32_t r = 0;
#pragma unroll 4
                for (uint32_t i = 0; i < m; ++i)
                    r += sm.cand[i] > c ? 1u : 0u;
                if (r == need - 1)
                    sm.kappa = c;
            }
        }
        __syncthreads();
    };
    uint32_t tau = 0u;                          // keys below it cannot be among the k largest
    if (!general && k <= (uint32_t)kT) {
        // 2a. the k-th largest of the threads' maxima (composites: unique)
        if (holds)
            atomicAdd(&sm.hist[bin_of(tmax)], 1u);
        __syncthreads();
        kth_bin(k);
        const uint32_t dt = sm.d, mt = sm.in_d, need_t = sm.need;
        if (dt != 0xFFFFFFFFu && mt <= (uint32_t)kCap) {
            if (holds && bin_of(tmax) == dt)
                sm.cand[atomicAdd(&sm.ncand, 1u)] = comp_key(tmax, (uint32_t)t);
            __syncthreads();
            rank_cand(mt, need_t);
            tau = (uint32_t)(sm.kappa >> 32);
        }
        sm.hist[t] = 0u;
        if (t == 0) {
            sm.ncand = 0u;
            sm.d = 0xFFFFFFFFu;
        }
        __syncthreads();
    }
    if (!general) {
        // 2. histogram of the keys >= tau (and their list, when kept)
        const bool keeping = keep != nullptr && tau != 0u;
        each_key([&](uint32_t key, uint32_t e) __attribute__((always_inline)) {
            if (key >= tau) {
                atomicAdd(&sm.hist[bin_of(key)], 1u);
                if (keeping) {
                    const uint32_t j = atomicAdd(&sm.nkeep, 1u);
                    if (j < keep_cap)
                        keep[j] = comp_key(key, e);
                }
            }
        });
        __syncthreads();
        kth_bin(k);
        const uint32_t d = sm.d, m = sm.in_d;
        general = d == 0xFFFFFFFFu || m > (uint32_t)kCap;
        if (!general) {
            // 3. keys above bin d are winners; bin d's entries are ranked
            auto mark = [&](uint32_t key, uint32_t e) __attribute__((always_inline)) {
                if (key >= tau) {
                    const uint32_t b = bin_of(key);
                    if (b > d)
                        atomicOr(&bitmap[e >> 5], 1u << (e & 31));
                    else if (b == d)
                        sm.cand[atomicAdd(&sm.ncand, 1u)] = comp_key(key, e);
                }
            };
            const uint32_t nkeep = sm.nkeep;
            if (keeping && nkeep <= keep_cap) {
                for (uint32_t j = t; j < nkeep; j += kT) {
                    const uint64_t c = keep[j];
                    mark((uint32_t)(c >> 32), ~(uint32_t)c);
                }
            } else {
                each_key(mark);
            }
            __syncthreads();
            rank_cand(m, sm.need);
            // 4. bin d's winners: its composites >= kappa
            const uint64_t kappa = sm.kappa;
            for (uint32_t j = t; j < m; j += kT) {
                const uint64_t c = sm.cand[j];
                if (c >= kappa) {
                    const uint32_t e = ~(uint32_t)c;
                    atomicOr(&bitmap[e >> 5], 1u << (e & 31));
                }
            }
            __syncthreads();
            emit_bitmap(sm, bitmap, nwords, k, emit);
            return;
        }
    }
    __syncthreads();
    general_path(a, sm, bitmap, lkeys, emit);
}

// ------------------------------------------------------------------ routine

// Whole workgroup (kT threads) calls; `lds` holds lds_bytes(a.nb) bytes.
// emit(slot, id) receives each of the k winners exactly once, slot = its rank
// in ascending id order.  Returns after the last emit of the calling thread;
// callers synchronise before reading what emit wrote.
template <class Emit>
__device__ void run(const SelectArgs &a, char *lds, Emit emit)
{
    Smem &sm = *reinterpret_cast<Smem *>(lds);
    const uint32_t k = (uint32_t)a.k;
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(lds + (sizeof(Smem) + 15) / 16 * 16);
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const uint32_t nchunks = (uint32_t)a.ntiles * (uint32_t)a.T / 2;
    // the lists decide only when they hold well over k entries: with fewer
    // than 4k the tiles' lists are full of winners and the check fails
    bool general = nchunks > (uint32_t)(kT * kChunks) || 2ull * nchunks < 4ull * k;

    // clear: histogram, bitmap words 2t and 2t+1, the counters
    sm.hist[t] = 0u;
    uint2 *own = reinterpret_cast<uint2 *>(bitmap) + t;
    *own = make_uint2(0u, 0u);
    if (t == 0) {
        sm.ncand = 0u;
        sm.bad = 0u;
    }

    // chunks t + 1024q of U (2 composites each), all loads in flight together
    // (no lists: the general path over the keys)
    general = general || !a.lists;
    uint64_t u[kEntries];
    if (!general) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.lists);
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const uint32_t c = (uint32_t)t + (uint32_t)(kT * q);
            const uint4 v = src[c < nchunks ? c : nchunks - 1];
            const bool in = c < nchunks;
            u[2 * q] = in ? ((uint64_t)v.y << 32) | v.x : 0ull;
            u[2 * q + 1] = in ? ((uint64_t)v.w << 32) | v.z : 0ull;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEntries; ++e)
            u[e] = 0ull;
    }
    // 1. key range of the listed entries (an empty slot has key 0: it wraps
    //    to the top in key - 1 and is the bottom for the maximum)
    uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int e = 0; e < kEntries; ++e) {
        const uint32_t key = (uint32_t)(u[e] >> 32);
        kmin1 = min(kmin1, key - 1u);
        kmax = max(kmax, key);
    }
    kmin1 = wave::reduce_min_u32(kmin1);
    kmax = wave::reduce_max_u32(kmax);
    if (lane == 0) {
        sm.rmin[wv] = kmin1;
        sm.rmax[wv] = kmax;
    }
    __syncthreads();                                                    // barrier
#pragma unroll
    for (int i = 0; i < kWaves; i += 4) {
        const uint4 a4 = reinterpret_cast<const uint4 *>(sm.rmin)[i / 4];
        const uint4 b4 = reinterpret_cast<const uint4 *>(sm.rmax)[i / 4];
        kmin1 = min(min(kmin1, a4.x), min(a4.y, min(a4.z, a4.w)));
        kmax = max(max(kmax, b4.x), max(b4.y, max(b4.z, b4.w)));
    }
    const uint32_t kmin = kmin1 + 1u;
    const float mn = key_score(kmin), mx = key_score(kmax);
    const float range = mx - mn;
    const float scale = (float)kBins / range;
    general = general || kmin1 == 0xFFFFFFFFu || kmin < kKeyFiniteLo || kmax > kKeyFiniteHi ||
              !(range > 0.0f) || !(range < __builtin_inff()) || !(scale < __builtin_inff());
    // All listed scores >= 0 (the usual case for the tiles' top entries): bins
    // linear in the key itself, which is linear in the score inside a binade;
    // otherwise linear in the score (the key space has a wide gap around 0).
    const bool by_key = kmin >= 0x80000000u;
    const int kshift = 32 - __clz((int)(kmax - kmin)) - 10;
    const uint32_t ksh = kshift > 0 ? (uint32_t)kshift : 0u;     // (kmax - kmin) >> ksh < 1024

    if (!general) {
        // 2. linear histogram; an empty slot (key 0) lands in bin 0, which the
        //    fast path never resolves (it falls back below), and is left out
        //    of the counts: its atomic would only add to bin 0's, and the
        //    empty slots of short lists (a few thousand at 64k contexts) all
        //    hitting one LDS address serialise for microseconds
        uint32_t bins[kEntries];
#pragma unroll
        for (int e = 0; e < kEntries; ++e) {
            const uint32_t key = (uint32_t)(u[e] >> 32);
            uint32_t b;
            if (by_key) {
                b = (key > kmin ? key - kmin : 0u) >> ksh;
            } else {
                const float s = fmaxf(key_score(key), mn);             // in [mn, mx]
                b = (uint32_t)((s - mn) * scale);                      // in [0, 1024]
                b = b < (uint32_t)kBins - 1 ? b : (uint32_t)kBins - 1;
            }
            bins[e] = b;
            if (key != 0u)
                atomicAdd(&sm.hist[b], 1u);
        }
        __syncthreads();                                                // barrier
        // the bin d holding the k-th largest: thread t takes bin 1023 - t, so a
        // prefix sum over threads is the count of entries in higher bins
        {
            const uint32_t h = sm.hist[kBins - 1 - t];
            const uint32_t incl = wave::incl_scan_add(h);
            if (lane == 63)
                sm.wtot[wv] = incl;
            __syncthreads();                                            // barrier
            uint32_t off = 0, tot = 0;
#pragma unroll
            for (int i = 0; i < kWaves; i += 4) {
                const uint4 w4 = reinterpret_cast<const uint4 *>(sm.wtot)[i / 4];
                tot += w4.x + w4.y + w4.z + w4.w;
                off += (i < wv ? w4.x : 0u) + (i + 1 < wv ? w4.y : 0u) +
                       (i + 2 < wv ? w4.z : 0u) + (i + 3 < wv ? w4.w : 0u);
            }
            const uint32_t above = off + incl - h;
            if (above < k && above + h >= k) {
                sm.d = (uint32_t)(kBins - 1 - t);
                sm.need = k - above;
                sm.in_d = h;
            }
            if (t == 0 && tot < k)
                sm.d = 0u;                                    // not found: general path
        }
        __syncthreads();                                                // barrier
        const uint32_t d = sm.d, m = sm.in_d;
        general = d == 0u || m > (uint32_t)kCap;

        if (!general) {
            // 3. the entries of bin d to LDS (empty slots sit in bin 0)
            uint32_t nd = 0;
#pragma unroll
            for (int e = 0; e < kEntries; ++e)
                nd += bins[e] == d ? 1u : 0u;
            if (nd) {
                uint32_t o = atomicAdd(&sm.ncand, nd);
#pragma unroll
                for (int e = 0; e < kEntries; ++e)
                    if (bins[e] == d)
                        sm.cand[o++] = u[e];
            }
            __syncthreads();                                            // barrier
            if (wv == 0) {
                // wave 0 ranks them by counting: kappa = the need-th largest
                const uint32_t need = sm.need;
                for (uint32_t j = lane; j < m; j += kWave) {
                    const uint64_t c = sm.cand[j];
                    uint32_t r = 0;
#pragma unroll 4
                    for (uint32_t i = 0; i < m; ++i)
                        r += sm.cand[i] > c ? 1u : 0u;
                    if (r == need - 1)
                        sm.kappa = c;
                }
            }
            __syncthreads();                                            // barrier
            const uint64_t kappa = sm.kappa;

            // 4. winners into the bitmap (straight from registers, no return
            //    values awaited); exactness check.  The last slot of a list is
            //    the odd entry of chunks c with (c+1) % (T/2) == 0, i.e. of
            //    every chunk of threads with (t+1) % (T/2) == 0.
            bool win[kEntries];
#pragma unroll
            for (int e = 0; e < kEntries; ++e)
                win[e] = u[e] >= kappa;
            const bool holds_last = (((uint32_t)t + 1) & ((uint32_t)a.T / 2 - 1)) == 0;
            bool bad = false;
#pragma unroll
            for (int q = 0; q < kChunks; ++q)
                bad = bad || (holds_last && win[2 * q + 1]);
#pragma unroll
            for (int e = 0; e < kEntries; ++e)
                if (win[e]) {
                    const uint32_t id = ~(uint32_t)u[e];
                    atomicOr(&bitmap[id >> 5], 1u << (id & 31));
                }
            if (bad)
                sm.bad = 1u;
            __syncthreads();                                            // barrier
            general = sm.bad != 0u;
            if (!general) {
                // 5. thread t owns bitmap words 2t, 2t+1 (ids 64t .. 64t+63):
                //    its first slot = winners in lower words, by a DPP scan in
                //    the wave plus the totals of the lower waves
                const uint2 wd = *own;
                const uint32_t pc = (uint32_t)(__popc(wd.x) + __popc(wd.y));
                const uint32_t wincl = wave::incl_scan_add(pc);
                if (lane == 63)
                    sm.wtot[wv] = wincl;
                __syncthreads();                                        // barrier
                const uint32_t wt = lane < kWaves ? sm.wtot[lane] : 0u;
                const uint32_t wexcl_all = wave::incl_scan_add(wt) - wt;
                uint32_t slot = wave::readlane(wexcl_all, wv) + wincl - pc;
                uint64_t bits = ((uint64_t)wd.y << 32) | wd.x;
                while (bits) {
                    const int b = __ffsll((long long)bits) - 1;
                    bits &= bits - 1;
                    if (slot < k)
                        emit(slot, 64u * (uint32_t)t + (uint32_t)b);
                    ++slot;
                }
                return;
            }
        }
    }

    // ---------------------------------------------------------- general path
    __syncthreads();
    keys_path(a, sm, bitmap, a.lkeys_off ? reinterpret_cast<uint32_t *>(lds + a.lkeys_off) : nullptr, emit);
}

}  // namespace sel
}  // namespace qsa
