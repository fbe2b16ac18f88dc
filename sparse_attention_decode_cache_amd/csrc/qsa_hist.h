// qsa_hist.h -- the global score histogram that lets every attention
// workgroup find the k-th largest block score without reading every tile's
// candidate list [post 10, "QSA indexer" and "block-domain top-k（COMMON-006）
// 実装は見送り": top-k over block scores].
//
// The score pass inserts every block whose score is >= L into kBins bins
// over the window [L, H] (scores >= H share the top bin) as soon as the
// block's score is known: per bin the count, the largest composite and the
// smallest (kept as the largest complement), all by atomics whose result
// nobody waits for.  If at least k blocks are >= L, the k-th largest
// composite kappa lies in the bin d where the count from the top reaches k;
// the counts of the bins at and above d are exact because every block >= L
// was inserted.  With `need` = how many of bin d win, kappa is bin d's
// smallest composite when all of them win and its largest when one does; any
// other split of a bin (rare: the bins are fine where kappa falls) and
// anything else the histogram cannot decide sends the call to the full top-k
// over every key.  A tile list of T entries can hide a winner only if its
// last entry is >= kappa: the maximum of those last entries (inside the
// window) must be below kappa.
//
// The bins are linear in the score in two pieces: kFine bins over [L, M)
// around where kappa is expected and the rest over [M, H).  The window comes
// from the query's score scale
//   sigma = sqrt(sum_h ||w_h q_h||^2 * mean_i gamma_i^2)
// (the spread of the scores of pooled rows with independent entries: RMSNorm
// leaves each entry of a row with mean square ~ gamma_i^2) and two ratios fed
// back by the previous call on the same workspace, its kappa / sigma and its
// top entry / sigma:  L = (rho_k - kBelow) sigma, M = (rho_k + kMid) sigma,
// H = (rho_top + kAbove) sigma.  A window that misses kappa only costs the
// full top-k for that call (and moves the next window).
//
// A window is taken from the fed-back ratios only when the feedback word says
// a merge wrote them (a fresh workspace holds whatever the memory held: its
// ratios could put L anywhere, and every block >= L is inserted); otherwise
// from defaults.  No kernel of the score pass writes that word or the ratios.
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
constexpr int kFine = kBins * 3 / 4;     // bins over [L, M)
constexpr int kLast = kHistLast;         // words holding the maximum of the tiles' last entries
constexpr uint64_t kTagClean = 0x5153412d48495354ull;   // low byte 0x54: never an epoch stamp
constexpr uint64_t kFeedback = 0x5153412d46454544ull;   // rho_k / rho_top were written by a merge
// Window margins in units of sigma.  kappa / sigma of independent queries
// over the same keys moves by about 0.02 from one call to the next.
constexpr float kBelow = 0.12f;
constexpr float kMid = 0.15f;
constexpr float kAbove = 0.5f;

__host__ __device__ inline uint64_t tag_ok(uint64_t epoch) { return (epoch << 8) | 0x11u; }
__host__ __device__ inline uint64_t tag_bad(uint64_t epoch) { return (epoch << 8) | 0x22u; }

// Control words at the start of the region.
struct Ctrl {
    uint64_t tag;       // kTagClean, or this call's tag_ok / tag_bad stamp
    uint64_t status;    // (epoch << 8) | path of the last decode step on this workspace
    float sigma;        // this call's score scale (written by score workgroup 0)
    float lo, mid, hi;  // this call's window pieces L, M, H (same)
    float rho_k, rho_top;   // the next call's kappa / sigma and top / sigma (written at the end)
    float inv1, inv2;   // this call's bin map: bins per unit score below and above M
    uint32_t klo, kmid, khi, map_ok;
    // what the attention kernel leaves for the merge kernel
    uint64_t kappa;     // the k-th largest composite (histogram path)
    uint32_t btop;      // the top nonempty bin (histogram path)
    uint32_t path;      // kPathFast or kPathFull
    uint32_t kmin, kmax;    // the smallest and largest chosen keys (full top-k)
    uint64_t fb;            // kFeedback once a merge has written rho_k / rho_top (else: defaults)
    uint32_t pad[40];
};
static_assert(sizeof(Ctrl) == 256, "one 256-byte line");

// Selection paths recorded in Ctrl::status.
constexpr uint32_t kPathFast = 1;        // histogram + own tile lists
constexpr uint32_t kPathFull = 2;        // the full top-k over every key

// Monotone map of an order-preserving score key >= key(L) to a bin.
struct Map {
    float lo, mid, inv1, inv2;
    uint32_t klo, kmid, khi;
    bool ok;
};

__device__ inline Map make_map(float L, float M, float H)
{
    Map m;
    m.lo = L;
    m.mid = M;
    m.inv1 = (float)kFine / (M - L);
    m.inv2 = (float)(kBins - 1 - kFine) / (H - M);
    m.klo = score_key(L);
    m.kmid = score_key(M);
    m.khi = score_key(H);
    m.ok = L > -3.0e38f && H < 3.0e38f && M > L && H > M && m.inv1 > 0.0f && m.inv1 < 3.0e38f &&
           m.inv2 > 0.0f && m.inv2 < 3.0e38f && m.klo < m.kmid && m.kmid < m.khi;
    return m;
}

// The map the score pass wrote into the control block.
__device__ inline Map stored_map(const Ctrl &c)
{
    Map m;
    m.lo = c.lo;
    m.mid = c.mid;
    m.inv1 = c.inv1;
    m.inv2 = c.inv2;
    m.klo = c.klo;
    m.kmid = c.kmid;
    m.khi = c.khi;
    m.ok = c.map_ok != 0u;
    return m;
}

// Whether the key is inside the window's reach (score >= L).
__device__ inline bool in_window(uint32_t key, const Map &m) { return key >= m.klo; }

// Bin of a key with in_window(key): fine bins [0, kFine) below M, coarse bins
// [kFine, kBins - 1) from M, the top bin from H.  Non-decreasing in the key.
__device__ inline uint32_t bin_of(uint32_t key, const Map &m)
{
    if (key >= m.khi)
        return (uint32_t)kBins - 1u;
    const float s = key_score(key);          // finite, in [L, H)
    if (key >= m.kmid) {
        const float x = (s - m.mid) * m.inv2;
        const uint32_t b = x > 0.0f ? (uint32_t)x : 0u;
        return (uint32_t)kFine + (b < (uint32_t)(kBins - 2 - kFine) ? b : (uint32_t)(kBins - 2 - kFine));
    }
    const float x = (s - m.lo) * m.inv1;
    const uint32_t b = x > 0.0f ? (uint32_t)x : 0u;
    return b < (uint32_t)kFine - 1u ? b : (uint32_t)kFine - 1u;
}

// Upper score edge of bin b (for the top-entry feedback; the top bin, open
// above, reports H plus the coarse range).
__device__ inline float bin_top(uint32_t b, const Map &m, float H)
{
    if (b >= (uint32_t)kBins - 1u)
        return H + (H - m.mid);
    if (b >= (uint32_t)kFine)
        return m.mid + (float)(b - kFine + 1u) / m.inv2;
    return m.lo + (float)(b + 1u) / m.inv1;
}

// The window of this call from the fed-back ratios (sanitised: a fresh or
// garbled control block gives the caller's defaults).
__device__ inline void window(float sigma, float rho_k, float rho_top, float def_k, float def_top,
                              float &L, float &M, float &H)
{
    const bool sane = rho_k > -1.0e4f && rho_k < 1.0e4f && rho_top >= rho_k && rho_top < rho_k + 1.0e4f;
    if (!sane) {
        rho_k = def_k;
        rho_top = def_top;
    }
    L = (rho_k - kBelow) * sigma;
    M = (rho_k + kMid) * sigma;
    const float top = rho_top + kAbove;
    H = (top > rho_k + kMid + kAbove ? top : rho_k + kMid + kAbove) * sigma;
}

}  // namespace hist
}  // namespace qsa
