// qsa_hist.h -- the global score histogram that lets every attention
// workgroup find the k-th largest block score without reading every tile's
// candidate list [post 10, "QSA indexer" and "block-domain top-k（COMMON-006）
// 実装は見送り": top-k over block scores].
//
// The score pass inserts the entries of each tile's list (its T largest
// composite keys) whose score is >= L into kBins bins LINEAR in the score
// over the window [L, H] (scores >= H share the top bin).  A bin's entries
// also go to its bucket (kCap slots; the slot is the count the atomic
// returned).  If at least k entries are >= L, the k-th largest composite
// kappa lies in the bin d where the count from the top reaches k and is the
// need-th largest of that bin's bucket; the counts of the bins at and above d
// are exact because every entry >= L was inserted.  A tile list of T entries
// can hide a winner only if its last entry is >= kappa: the maximum of those
// last entries (>= L) must fall in a bin below d.  Anything the histogram
// cannot decide sends the call to the full top-k over every key.
//
// The window is set per call from the query's score scale
//   sigma = sqrt(sum_h ||w_h q_h||^2 * mean_i gamma_i^2)
// (the spread of the scores of pooled rows with independent entries: RMSNorm
// leaves each entry of a row with mean square ~ gamma_i^2) as
// [rho_lo sigma, rho_hi sigma], where rho_lo, rho_hi are fed back by the
// previous call on the same workspace: kappa / sigma minus a margin, and the
// top entry / sigma plus a margin.  A window that misses kappa only costs
// the full top-k for that call (and moves the next window).  So only the
// few entries near the top are inserted and the bins are fine there: the
// device atomics seldom meet on one address.
//
// Consistency: the histogram region is trusted only when its tag says the
// previous call cleared it.  The score pass's workgroup 0 reads the tag and
// stamps it with this call's epoch, marked clean-start or not; the attention
// kernel requires the clean-start stamp of its own epoch, and the merge
// kernel after it clears the region and writes the clean tag.
#pragma once
#include "qsa_internal.h"

namespace qsa {
namespace hist {

constexpr int kBins = kHistBins;
constexpr int kCap = kHistCap;           // bucket slots per bin
constexpr int kLast = kHistLast;         // words holding the maximum of the tiles' last entries
constexpr uint64_t kTagClean = 0x5153412d48495354ull;   // low byte 0x54: never an epoch stamp

__host__ __device__ inline uint64_t tag_ok(uint64_t epoch) { return (epoch << 8) | 0x11u; }
__host__ __device__ inline uint64_t tag_bad(uint64_t epoch) { return (epoch << 8) | 0x22u; }

// Control words at the start of the region.
struct Ctrl {
    uint64_t tag;       // kTagClean, or this call's tag_ok / tag_bad stamp
    uint64_t status;    // (epoch << 8) | path of the last decode step on this workspace
    float sigma;        // this call's score scale (written by score workgroup 0)
    float lo, hi;       // this call's window [L, H] (same)
    float rho_lo, rho_hi;   // the next call's window in units of its sigma (written at the end)
    float inv;          // this call's bin map: kBins / (H - L), key(L), key(H), map usable
    uint32_t klo, khi, map_ok;
    // what the attention kernel leaves for the merge kernel
    uint64_t kappa;     // the k-th largest composite (histogram path)
    uint32_t btop;      // the top nonempty bin (histogram path)
    uint32_t path;      // kPathFast or kPathFull
    uint32_t kmin, kmax;    // the smallest and largest chosen keys (full top-k)
    uint32_t pad[44];
};
static_assert(sizeof(Ctrl) == 256, "one 256-byte line");

// Selection paths recorded in Ctrl::status.
constexpr uint32_t kPathFast = 1;        // histogram + own tile lists
constexpr uint32_t kPathFull = 2;        // the full top-k over every key

// Monotone map of an order-preserving score key >= key(L) to a bin.
struct Map {
    float lo, inv;
    uint32_t klo, khi;
    bool ok;
};

__device__ inline Map make_map(float L, float H)
{
    Map m;
    m.lo = L;
    m.inv = (float)kBins / (H - L);
    m.klo = score_key(L);
    m.khi = score_key(H);
    m.ok = L > -3.0e38f && H < 3.0e38f && H > L && m.inv > 0.0f && m.inv < 3.0e38f;
    return m;
}

// The map the score pass wrote into the control block.
__device__ inline Map stored_map(const Ctrl &c)
{
    Map m;
    m.lo = c.lo;
    m.inv = c.inv;
    m.klo = c.klo;
    m.khi = c.khi;
    m.ok = c.map_ok != 0u;
    return m;
}

// Whether the key is inside the window's reach (score >= L).
__device__ inline bool in_window(uint32_t key, const Map &m) { return key >= m.klo; }

// Bin of a key with in_window(key): linear in the score, the top bin also
// takes every score >= H.
__device__ inline uint32_t bin_of(uint32_t key, const Map &m)
{
    if (key >= m.khi)
        return (uint32_t)kBins - 1u;
    const float s = key_score(key);          // finite, in [L, H)
    const float x = (s - m.lo) * m.inv;
    const uint32_t b = x > 0.0f ? (uint32_t)x : 0u;
    return b < (uint32_t)kBins - 1u ? b : (uint32_t)kBins - 1u;
}

// The window of this call from the fed-back ratios (sanitised: a fresh or
// garbled control block gives the caller's defaults).
__device__ inline void window(float sigma, float rho_lo, float rho_hi, float def_lo, float def_hi,
                              float &L, float &H)
{
    const bool sane = rho_lo > -1.0e4f && rho_lo < 1.0e4f && rho_hi > rho_lo + 1.0e-3f &&
                      rho_hi < rho_lo + 1.0e4f;
    if (!sane) {
        rho_lo = def_lo;
        rho_hi = def_hi;
    }
    L = rho_lo * sigma;
    H = rho_hi * sigma;
}

}  // namespace hist
}  // namespace qsa
