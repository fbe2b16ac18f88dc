// k_decode.hip -- stages 3 and 4 of the decode step in two kernels, after a
// score pass that put its tile lists into the global histogram (qsa_hist.h).
//
// [post 10, "QSA indexer": the top 2048 tokens (512 blocks) by block score;
//  "block-domain top-k（COMMON-006）実装は見送り": top-k over block scores,
//  the chosen blocks expanded to cells, the tail appended;
//  "selected QSA K/V gather（COMMON-005）": attention over those cells only.]
//
// Grid (ns splits, kv_heads), 1024 threads, one workgroup per CU.  Split s
// owns the score tiles [s ntiles / ns, (s + 1) ntiles / ns) and attends the
// cells of the winners among its tiles' list entries.  The kernel is bound by
// latency, and with 16 waves on a CU every instruction all of them execute
// costs 16 cycles, so each phase runs on the waves that need it:
//   1. one round of loads: thread t < 512 four bins of the histogram
//      (count and extremes, top bins first) and the split's list entries t
//      and 512 + t; wave 8 the tiles' last-entry maxima; waves 8-15 the q
//      operand;
//   2. a prefix sum over the threads finds the bin d holding the k-th
//      largest entry, how many of bin d win (`need`), kappa from the bin's
//      extremes and the top nonempty bin;
//   3. the split's entries >= kappa win: they go to its block list (ballot
//      compaction), and the last split adds its tail cells 4 nb + j
//      (j < n mod 4) as a block of their own;
//   4. 16 threads per cell load its K and V rows (one address per thread);
//      K and V land in separate LDS tiles;
//   5. a wave per 16 cells takes their G logits on the matrix cores (q as
//      f16 hi + lo); waves h < G run the online softmax of head h; every wave takes
//      P.V for its 16-dim output tiles on the matrix cores (passes of up to
//      64 cells, k-steps only over the pass's cells);
//   6. the partial (acc, m, l) and, when the ids are wanted, the split's
//      winners go out with plain stores.
// The merge kernel after it takes one (query head, 64-dim slice) per
// workgroup, and one more workgroup feeds kappa and the top score back as
// the next call's window, clears the histogram and gathers the splits'
// winners in order.  (Merging inside the attention kernel, behind flags the
// splits publish, was measured slower on gfx950: coherent stores, their
// waits and the polling cost more than a kernel boundary.)
// The histogram decides exactly when its region started this call cleared,
// at least k entries reached the window, bin d is split all-or-one (so that
// its extremes give kappa) and no tile list can hide a winner (the largest
// last entry of a full list is below kappa).  Otherwise every
// workgroup runs the full top-k of qsa_select.h over the keys and takes an
// even share of the chosen blocks.  No workgroup waits on another.
#include "qsa_hist.h"
#include "qsa_internal.h"
#include "qsa_select.h"
#include "qsa_unit.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

constexpr int kNT = kDecodeThreads;
constexpr int kNW = kNT / kWave;
constexpr int kNA = kNT / 2;                     // threads that attend (waves 0-7)
constexpr int kNAW = kNA / kWave;
constexpr int kPC = 64;                          // cells per pass (two per 16 threads)
constexpr int kMaxOwn = kNT;                     // blocks a split attends at most
static_assert(kNT == sel::kT, "the full top-k runs in the same workgroup");
static_assert(hist::kBins == 4 * kNA, "thread t < 512 scans four bins");
static_assert(kNW == 16 && kNAW == 8 && kPC == 2 * (kNA / 16), "wave counts the phases assume");
static_assert(offsetof(hist::Ctrl, status) == QSA_DECODE_STATUS_OFFSET && hist::kPathFast == QSA_PATH_HIST &&
                  hist::kPathFull == QSA_PATH_FULL,
              "the status word as the header documents it");
// The full top-k's LDS for up to 2^19 blocks (it overlays the K / V tiles).
constexpr size_t kFullLds = (sizeof(sel::Smem) + 15) / 16 * 16 + 4 * ((size_t)1 << 19) / 32;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

template <int DH>
struct DecShape {
    static constexpr int KS = DH / 32;           // MFMA k-steps of a row
    static constexpr int KROW = 2 * DH + 16;     // padded LDS bytes of a K or V row
    static constexpr int CH = DH / 8;            // 16-byte chunks of a row
    static constexpr int CPT = (CH + 15) / 16;   // chunks per thread (16 threads per cell)
    static constexpr int NT = DH / 16;           // 16-dim output tiles of P.V
    static constexpr int TPW = (NT + kNAW - 1) / kNAW;
    static constexpr size_t TILE = (size_t)kPC * KROW;
};

template <int DH, int G>
struct DecLds {
    using S = DecShape<DH>;
    static constexpr size_t kTiles = 2 * S::TILE > kFullLds ? 2 * S::TILE : kFullLds;
    alignas(16) unsigned char tiles[kTiles];     // K tile, V tile (or the full top-k's scratch)
    alignas(16) uint4 qb[S::KS][2][kWave];
    float lg[kPC][G + 1];
    // softmax weights, hi and lo halves, [head][cell]: rows padded by 16
    // bytes, so that the heads of one P.V operand read fall 4 banks apart
    alignas(16) _Float16 pt[2][G][kPC + 8];
    float sc[G];
    int32_t ids[kMaxOwn + 1];                    // the split's blocks (and the tail)
    alignas(16) uint32_t wcnt[2 * kNAW];         // winners per wave, entries t and 512 + t
    alignas(16) uint32_t wtot[kNW];              // histogram counts per wave (waves 0-7)
    uint32_t d, need, in_d, found, nown, btop, kmin_w, kmax_w;
    uint64_t kappa, lastmax;
};

// The K and V chunks of one cell a thread loads: chunks sub + 16 j of the
// cell's rows (returned by value, so they stay in registers).
template <int N>
struct RowChunks {
    uint4 k[N], v[N];
};

template <int DH>
__device__ inline RowChunks<DecShape<DH>::CPT> load_rows(const DecodeArgs &a, const int32_t *ids, int ncell,
                                                         int c, int sub, int g)
{
    using S = DecShape<DH>;
    RowChunks<S::CPT> r;
    if (c < ncell) {
        const int32_t b = ids[c >> 2];
        const size_t row = ((size_t)(4 * (int64_t)b + (c & 3)) * a.kv_heads + (size_t)g) * DH;
        const uint4 *kp = reinterpret_cast<const uint4 *>(a.k + row);
        const uint4 *vp = reinterpret_cast<const uint4 *>(a.v + row);
#pragma unroll
        for (int j = 0; j < S::CPT; ++j)
            if (sub + 16 * j < S::CH) {
                r.k[j] = kp[sub + 16 * j];
                r.v[j] = vp[sub + 16 * j];
            }
    }
    return r;
}

// Cell `lc` of a pass into the LDS tiles.  V rows of cells that do not count
// (past the pass's cells, up to the last k-step, and the tail block's cells
// past the tail) are zeroed: their weight is 0, and 0 times whatever is there
// could be NaN; their K rows are left alone (those logits become -inf).
// The tiles' 16-byte chunk c of row r sits at chunk c ^ tswz(r): a P.V
// operand read takes one 2-byte column of rows 8 kq + e (kq < 4, e < 8), and
// with rows 2 DH + 16 bytes apart those four row groups would share banks;
// the swizzle puts them 32 bytes apart.  Every access to the K and V tiles
// goes through it.
__device__ __forceinline__ int tswz(int r) { return 2 * ((r >> 3) & 3); }

template <int DH, int CPT>
__device__ inline void put_rows(unsigned char *ktile, unsigned char *vtile, const RowChunks<CPT> &kv, int lc,
                                int sub, bool live)
{
    using S = DecShape<DH>;
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (sub + 16 * j < S::CH) {
            const int off = lc * S::KROW + 16 * ((sub + 16 * j) ^ tswz(lc));
            if (live)
                *(uint4 *)(ktile + off) = kv.k[j];
            *(uint4 *)(vtile + off) = live ? kv.v[j] : make_uint4(0u, 0u, 0u, 0u);
        }
}

// Sum of v[i] over i < n (n <= 16, wave-uniform) of 16 words read as uint4.
__device__ inline uint32_t sum_below(const uint32_t *v, int n)
{
    const uint4 *v4 = reinterpret_cast<const uint4 *>(v);
    uint32_t s = 0;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const uint4 x = v4[q4];
        s += (4 * q4 + 0 < n ? x.x : 0u) + (4 * q4 + 1 < n ? x.y : 0u) + (4 * q4 + 2 < n ? x.z : 0u) +
             (4 * q4 + 3 < n ? x.w : 0u);
    }
    return s;
}

template <int DH, int G>
__global__ __launch_bounds__(kNT) void k_decode_attend(DecodeArgs a)
{
    using S = DecShape<DH>;
    constexpr int KS = S::KS, KROW = S::KROW, CPT = S::CPT, NT = S::NT, TPW = S::TPW;
    extern __shared__ uint4 dec_lds[];
    DecLds<DH, G> &L = *reinterpret_cast<DecLds<DH, G> *>(dec_lds);
    unsigned char *ktile = L.tiles, *vtile = L.tiles + S::TILE;
    const int t = threadIdx.x, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int s = blockIdx.x, g = blockIdx.y;
    const int ns = a.ns;
    const int T = a.sa.T;
    const int64_t ntl = a.sa.ntiles;
    const int tile0 = (int)((int64_t)s * ntl / ns), tile1 = (int)((int64_t)(s + 1) * ntl / ns);
    const int nent = (tile1 - tile0) * T;          // <= kNT (the launcher checks)
    const uint32_t k = (uint32_t)a.k_blocks;
    hist::Ctrl *ctrl = reinterpret_cast<hist::Ctrl *>(a.ctrl);

    // ---- 1. first-round loads, by role
    const uint64_t tag = ctrl->tag;
    const hist::Map map = hist::stored_map(*ctrl);
    // waves 0-7, thread t: bins b0 + 3 .. b0 (b0 = 2044 - 4t), so that
    // counts summed over threads in order run from the top bin down
    const int b0 = hist::kBins - 4 - 4 * t;
    uint4 hc = make_uint4(0u, 0u, 0u, 0u);
    ulonglong2 mx01{}, mx23{}, mn01{}, mn23{};
    uint64_t ent0 = 0, ent1 = 0;                    // list entries t and 512 + t
    if (t < kNA) {
        hc = *reinterpret_cast<const uint4 *>(a.hist + b0);
        mx01 = *reinterpret_cast<const ulonglong2 *>(a.bmax + b0);
        mx23 = *reinterpret_cast<const ulonglong2 *>(a.bmax + b0 + 2);
        mn01 = *reinterpret_cast<const ulonglong2 *>(a.bminc + b0);
        mn23 = *reinterpret_cast<const ulonglong2 *>(a.bminc + b0 + 2);
        if (t < nent)
            ent0 = a.sa.lists[(size_t)tile0 * T + t];
        if (kNA + t < nent)
            ent1 = a.sa.lists[(size_t)tile0 * T + kNA + t];
    }
    uint64_t lm = wv == 8 ? a.last[lane] : 0ull;
    if (t >= kNA) {
        // q of the group's G heads as the logit MFMA's B operand: slot x =
        // (k-step, lane) holds q[head x % 16][32 ks + 8 (x % 64 / 16) .. +8],
        // zero past G, as f16 hi and lo halves
        const int x = t - kNA;
        if (x < KS * kWave) {
            const int ks = x / kWave, l = x % kWave, hq = l % 16, d0 = 32 * ks + 8 * (l / 16);
            float4 u = make_float4(0.0f, 0.0f, 0.0f, 0.0f), v = u;
            if (hq < G) {
                const float *qp = a.q + ((size_t)g * G + hq) * DH + d0;
                u = *(const float4 *)qp;
                v = *(const float4 *)(qp + 4);
            }
            const float qf[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
            half8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                hi[j] = (_Float16)qf[j];
                lo[j] = (_Float16)(qf[j] - (float)hi[j]);
            }
            __builtin_memcpy(&L.qb[ks][0][l], &hi, 16);
            __builtin_memcpy(&L.qb[ks][1][l], &lo, 16);
        }
    }

    // ---- 2. waves 0-7: counts from the top (wave prefix sums, then the
    //         waves before); the thread whose bins reach k finds bin d, how
    //         many of it win (`need`) and kappa from the bin's extremes;
    //         wave 8: the largest last entry
    uint32_t cnt = 0, incl = 0;
    if (t < kNA) {
        cnt = hc.x + hc.y + hc.z + hc.w;
        incl = wave::incl_scan_add(cnt);
        if (lane == 63)
            L.wtot[wv] = incl;
    } else if (wv == 8) {
        lm = wave::reduce_max_u64(lm);
        if (lane == 0)
            L.lastmax = lm;
    }
    if (t == 0) {
        L.found = 0u;
        L.btop = 0u;
        L.kappa = ~0ull;
        L.kmin_w = 0xFFFFFFFFu;
        L.kmax_w = 0u;
    }
    __syncthreads();                                                    // barrier
    if (t < kNA) {
        const uint32_t above = incl - cnt + sum_below(L.wtot, wv);
        const uint32_t hv[4] = {hc.x, hc.y, hc.z, hc.w};
        const uint64_t mx[4] = {mx01.x, mx01.y, mx23.x, mx23.y};
        const uint64_t mnc[4] = {mn01.x, mn01.y, mn23.x, mn23.y};
        if (above == 0 && cnt > 0) {
            uint32_t bt = (uint32_t)b0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (hv[j] != 0u)
                    bt = (uint32_t)(b0 + j);
            L.btop = bt;
        }
        if (above < k && above + cnt >= k) {
            uint32_t acc = above, dd = 0, nd = 0, id = 0;
            uint64_t kx = 0;
            bool seek = true;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (seek && acc + hv[j] >= k) {
                    dd = (uint32_t)(b0 + j);
                    nd = k - acc;
                    id = hv[j];
                    // all of bin d win: kappa is its smallest; one wins: its
                    // largest; any other split is left to the full top-k
                    kx = nd == id ? ~mnc[j] : mx[j];
                    seek = false;
                }
                acc += hv[j];
            }
            L.d = dd;
            L.need = nd;
            L.in_d = id;
            L.kappa = kx;
            L.found = (nd == id || nd == 1u) ? 1u : 2u;
        }
    }
    __syncthreads();                                                    // barrier
    const uint64_t kappa = L.kappa;
    // a list of T entries hides no winner when its last entry is below kappa
    const bool fast = tag == hist::tag_ok(a.epoch) && L.found == 1u && map.ok && L.lastmax < kappa;
    // the last split also takes the tail cells 4 nb + j (j < n_tail) as a
    // block of its own (id nb)
    const bool tail_here = s == ns - 1 && a.n_tail > 0;

    // ---- 3. the split's blocks: its list entries >= kappa (the winners), in
    //         list order (ballot compaction); or the full top-k, split s
    //         taking the chosen slots [s per, s per + per).  From here on
    //         waves 0-7 carry on alone (the rest end: barriers then count
    //         only the waves still running).
    if (fast) {
        if (wv >= kNAW)
            return;
        const bool m0 = ent0 != 0ull && ent0 >= kappa, m1 = ent1 != 0ull && ent1 >= kappa;
        const uint64_t bal0 = __ballot(m0), bal1 = __ballot(m1);
        const uint32_t p0 = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal0, 0u));
        const uint32_t p1 = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal1, 0u));
        if (lane == 0) {
            L.wcnt[wv] = (uint32_t)__popcll(bal0);
            L.wcnt[kNAW + wv] = (uint32_t)__popcll(bal1);
        }
        __syncthreads();                                                // barrier
        const uint32_t tot0 = sum_below(L.wcnt, kNAW);
        if (m0)
            L.ids[sum_below(L.wcnt, wv) + p0] = (int32_t)(~(uint32_t)ent0);
        if (m1)
            L.ids[tot0 + sum_below(L.wcnt + kNAW, wv) + p1] = (int32_t)(~(uint32_t)ent1);
        if (t == 0) {
            uint32_t tot = tot0 + sum_below(L.wcnt + kNAW, kNAW);
            if (tail_here)
                L.ids[tot++] = a.nb;
            L.nown = tot;
        }
        __syncthreads();                                                // barrier
    } else {
        const uint32_t per = (k + (uint32_t)ns - 1u) / (uint32_t)ns;
        const uint32_t s0 = (uint32_t)s * per;
        int32_t *all = (s == 0 && g == 0) ? a.sel_out : nullptr;
        int32_t *ids = L.ids;
        const uint32_t *keys = (s == ns - 1 && g == a.kv_heads - 1) ? a.sa.keys : nullptr;   // the window feedback
        uint32_t *kmin = &L.kmin_w, *kmax = &L.kmax_w;
        sel::run(a.sa, reinterpret_cast<char *>(L.tiles), [=](uint32_t slot, uint32_t id) {
            if (slot - s0 < per)
                ids[slot - s0] = (int32_t)id;
            if (all)
                all[slot] = (int32_t)id;
            if (keys) {
                const uint32_t key = keys[id];
                atomicMin(kmin, key);
                atomicMax(kmax, key);
            }
        });
        if (t == 0) {
            uint32_t tot = s0 < k ? (k - s0 < per ? k - s0 : per) : 0u;
            if (tail_here)
                L.ids[tot++] = a.nb;
            L.nown = tot;
        }
        __syncthreads();                                                // barrier
        if (wv >= kNAW)
            return;
    }
    const uint32_t nown = L.nown;
    const int ncell = 4 * (int)nown;
    const int npass = (ncell + kPC - 1) / kPC;

    // ---- 4. K / V rows of the split's cells: thread t takes cells t / 16 and
    //         t / 16 + 32 of the pass, 16-byte chunks (t % 16) + 16 j of each
    //         one's K and V rows
    const int lc = t >> 4, sub = t & 15;
    RowChunks<CPT> kv0 = load_rows<DH>(a, L.ids, ncell, lc, sub, g);
    RowChunks<CPT> kv1 = load_rows<DH>(a, L.ids, ncell, lc + kPC / 2, sub, g);

    // ---- 5. attention in passes of up to 64 cells
    const int hn = lane & 15, kq = lane >> 4;
    float4v acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
        acc[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;          // wave h < G: head h
    for (int p = 0; p < npass; ++p) {
        const int np = ncell - kPC * p < kPC ? ncell - kPC * p : kPC;   // cells of this pass
        const int nks = (np + 31) / 32;                                  // P.V k-steps
        const int c0 = kPC * p + lc, c1 = c0 + kPC / 2;
        if (lc < 32 * nks)
            put_rows<DH, CPT>(ktile, vtile, kv0, lc, sub,
                              lc < np && !(L.ids[c0 >> 2] == a.nb && (lc & 3) >= a.n_tail));
        if (lc + kPC / 2 < 32 * nks)
            put_rows<DH, CPT>(ktile, vtile, kv1, lc + kPC / 2, sub,
                              lc + kPC / 2 < np && !(L.ids[c1 >> 2] == a.nb && (lc & 3) >= a.n_tail));
        // the next pass's rows load while this one computes (the registers
        // are free once the rows are in the tiles)
        if (p + 1 < npass) {
            kv0 = load_rows<DH>(a, L.ids, ncell, kPC * (p + 1) + lc, sub, g);
            kv1 = load_rows<DH>(a, L.ids, ncell, kPC * (p + 1) + lc + kPC / 2, sub, g);
        }
        __syncthreads();                                                // barrier: tiles
        if (wv < (np + 15) / 16) {
            // D[cell][head] = K[cell][:] . q[head][:], 16 cells per wave
            const int mc = lane & 15, kg = lane >> 4;
            float4v dd = {0.0f, 0.0f, 0.0f, 0.0f}, de = dd;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                half8 av, bh, bl;
                __builtin_memcpy(&av, ktile + (16 * wv + mc) * KROW + 16 * ((4 * ks + kg) ^ tswz(16 * wv + mc)), 16);
                __builtin_memcpy(&bh, &L.qb[ks][0][lane], 16);
                __builtin_memcpy(&bl, &L.qb[ks][1][lane], 16);
                dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, dd, 0, 0, 0);
                de = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, de, 0, 0, 0);
            }
            if (mc < G) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cl = 16 * wv + 4 * kg + j;
                    const int b = (kPC * p + cl) >> 2;
                    const bool valid = cl < np && !(L.ids[b] == a.nb && (cl & 3) >= a.n_tail);
                    L.lg[cl][mc] = valid ? a.scale * (dd[j] + de[j]) : -INFINITY;
                }
            }
        }
        __syncthreads();                                                // barrier: logits
        if (wv < G) {
            // online softmax of head `wv` over the pass's cells (lane = cell)
            const float xv = lane < np ? L.lg[lane][wv] : -INFINITY;
            const float mn = fmaxf(m_run, wave::reduce_max_f(xv));
            float scl = 1.0f, pv = 0.0f;
            if (mn != -INFINITY) {
                scl = m_run == -INFINITY ? 0.0f : expf(m_run - mn);
                pv = xv == -INFINITY ? 0.0f : expf(xv - mn);
            }
            l_run = l_run * scl + wave::reduce_add_f(pv);
            m_run = mn;
            const _Float16 ph = (_Float16)pv;
            L.pt[0][wv][lane] = ph;
            L.pt[1][wv][lane] = (_Float16)(pv - (float)ph);
            if (lane == 0)
                L.sc[wv] = scl;
        }
        __syncthreads();                                                // barrier: weights
        // out^T = out^T * sc + V^T P: A = 16 dims x 32 cells read down the V
        // tile's columns, B = 32 cells x 16 heads (zero past G), hi and lo
        const float scl = hn < G ? L.sc[hn] : 1.0f;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] *= scl;
        for (int ks = 0; ks < nks; ++ks) {
            half8 bh = {}, bl = {};
            if (hn < G) {
                __builtin_memcpy(&bh, &L.pt[0][hn][32 * ks + 8 * kq], 16);
                __builtin_memcpy(&bl, &L.pt[1][hn][32 * ks + 8 * kq], 16);
            }
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tile = wv + kNAW * i;
                if (NT % kNAW == 0 || tile < NT) {
                    // av[e] = V[32 ks + 8 kq + e][16 tile + hn] by two transpose
                    // reads (rows 32 ks + 8 kq + e: tswz = 2 kq for every e)
                    half8 av;
                    const unsigned char *p0 = vtile + (32 * ks + 8 * kq + (hn >> 2)) * KROW +
                                              16 * ((2 * tile + ((hn & 3) >> 1)) ^ (2 * kq)) + 8 * (hn & 1);
                    unit::lds_tr4(p0, av, 0);
                    unit::lds_tr4(p0 + 4 * KROW, av, 4);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bh, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bl, acc[i], 0, 0, 0);
                }
            }
        }
        if (p + 1 < npass)
            __syncthreads();                                            // barrier: tiles free
    }

    // ---- 6. the partial (acc[G][Dh], m[G], l[G]) and, when the ids are
    //         wanted, the split's winners (ascending); what the merge kernel
    //         needs of the selection goes to the control block
    const int64_t ps = dec_part_stride(G, DH);
    float *part = a.part + ((size_t)g * ns + s) * ps;
    if (hn < G) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wv + kNAW * i;
            if (NT % kNAW != 0 && tile >= NT)
                continue;
            *(float4v *)(part + hn * DH + 16 * tile + 4 * kq) = acc[i];
        }
    }
    if (wv < G && lane == 0) {
        part[G * DH + wv] = m_run;
        part[G * DH + G + wv] = l_run;
    }
    if (fast && a.sel_out && g == 0) {
        // the split's winners ascending: each one's rank among them (every
        // listed block but the tail wins)
        for (uint32_t j = (uint32_t)t; j < nown; j += kNA) {
            const int32_t id = L.ids[j];
            if (id == a.nb)
                continue;
            uint32_t r = 0;
            for (uint32_t i = 0; i < nown; ++i)
                r += (L.ids[i] != a.nb && L.ids[i] < id) ? 1u : 0u;
            a.stage[(size_t)s * k + r] = id;
        }
        if (t == 0)
            a.stage_n[s] = (int32_t)nown - (tail_here ? 1 : 0);
    }
    if (t == 0 && s == 0 && g == 0) {
        ctrl->path = fast ? hist::kPathFast : hist::kPathFull;
        ctrl->kappa = kappa;
        ctrl->btop = L.btop;
    }
    if (!fast && t == 0 && s == ns - 1 && g == a.kv_heads - 1) {
        ctrl->kmin = L.kmin_w;
        ctrl->kmax = L.kmax_w;
    }
}

// The merge of the splits' partials, after the attention kernel: workgroup
// (query head h, 64-dim slice ds) writes out[h][64 ds .. +64).  Thread t takes
// 4 dims (t % 16) of splits t / 16 and t / 16 + 64; wave 0 takes every
// split's m and l and turns the m's into weights once.  One more workgroup
// (the last) feeds kappa and the top score back as the next call's window,
// clears the histogram for the next call and, with ids wanted, gathers the
// splits' winners in order.
template <int DH, int G>
struct MergeLds {
    float mw[2 * kWave];                         // split weights
    float ltot;
    alignas(16) float macc[kNW][kWave];
    uint32_t wtot[kNW];
};

template <int DH, int G>
__global__ __launch_bounds__(kNT) void k_decode_merge(DecodeArgs a)
{
    static_assert(kDecodeMaxSplits <= 2 * kWave, "wave 0 holds two splits a lane");
    __shared__ MergeLds<DH, G> L;
    constexpr int kSlices = DH / kWave;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int ns = a.ns;
    const int nmu = a.kv_heads * G * kSlices;
    if ((int)blockIdx.x < nmu) {
        const int h = (int)blockIdx.x / kSlices, ds = (int)blockIdx.x % kSlices;
        const int g = h / G, hh = h % G;
        const int64_t ps = dec_part_stride(G, DH);
        const float *base = a.part + (size_t)g * ns * ps;
        const int q4 = 4 * (t & 15);
        const int sp0 = t >> 4, sp1 = sp0 + 64;
        const size_t aoff = (size_t)hh * DH + 64 * ds + q4;
        float4v x0 = {0.0f, 0.0f, 0.0f, 0.0f}, x1 = x0;
        if (sp0 < ns)
            x0 = *(const float4v *)(base + (size_t)sp0 * ps + aoff);
        if (sp1 < ns)
            x1 = *(const float4v *)(base + (size_t)sp1 * ps + aoff);
        if (wv == 0) {
            float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f;
            if (lane < ns) {
                m0 = base[(size_t)lane * ps + G * DH + hh];
                l0 = base[(size_t)lane * ps + G * DH + G + hh];
            }
            if (lane + 64 < ns) {
                m1 = base[(size_t)(lane + 64) * ps + G * DH + hh];
                l1 = base[(size_t)(lane + 64) * ps + G * DH + G + hh];
            }
            const float M = wave::reduce_max_f(fmaxf(m0, m1));
            const float w0 = m0 == -INFINITY ? 0.0f : expf(m0 - M);
            const float w1 = m1 == -INFINITY ? 0.0f : expf(m1 - M);
            L.mw[lane] = w0;
            L.mw[lane + 64] = w1;
            const float ls = wave::reduce_add_f(fmaf(w0, l0, w1 * l1));
            if (lane == 0)
                L.ltot = ls;
        }
        __syncthreads();
        const float w0 = L.mw[sp0], w1 = L.mw[sp1];
        float4v acc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j] = fmaf(w0, x0[j], w1 * x1[j]);
        // sum over the wave's four splits (lanes 16 apart), then over the waves
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[j] += __shfl_xor(acc[j], 16);
            acc[j] += __shfl_xor(acc[j], 32);
        }
        if (lane < 16)
            *(float4v *)&L.macc[wv][q4] = acc;
        __syncthreads();
        if (wv == 0) {
            float A = L.macc[0][lane];
#pragma unroll
            for (int w = 1; w < kNW; ++w)
                A += L.macc[w][lane];
            a.out[(size_t)h * DH + 64 * ds + lane] = A / L.ltot;
        }
        return;
    }

    // the bookkeeping workgroup
    hist::Ctrl *ctrl = reinterpret_cast<hist::Ctrl *>(a.ctrl);
    const bool fast = ctrl->path == hist::kPathFast;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    if (t < hist::kBins / 4)
        reinterpret_cast<uint4 *>(const_cast<uint32_t *>(a.hist))[t] = z;
    if (t < hist::kBins / 2) {
        reinterpret_cast<uint4 *>(const_cast<uint64_t *>(a.bmax))[t] = z;
        reinterpret_cast<uint4 *>(const_cast<uint64_t *>(a.bminc))[t] = z;
    }
    if (t < hist::kLast / 2)
        reinterpret_cast<uint4 *>(const_cast<uint64_t *>(a.last))[t] = z;
    if (t == 0) {
        // the next call's window: this call's kappa / sigma and top entry /
        // sigma (the histogram path knows the top only to its bin)
        const hist::Map map = hist::stored_map(*ctrl);
        const float sigma = ctrl->sigma;
        float kk, ktop;
        if (fast) {
            kk = key_score((uint32_t)(ctrl->kappa >> 32));
            ktop = hist::bin_top(ctrl->btop, map, ctrl->hi);
        } else {
            kk = key_score(ctrl->kmin);
            ktop = key_score(ctrl->kmax);
        }
        ctrl->rho_k = kk / sigma;       // NaN when sigma is 0 or not finite: defaults next time
        ctrl->rho_top = (ktop > kk ? ktop : kk) / sigma;
        ctrl->fb = hist::kFeedback;
        ctrl->tag = hist::kTagClean;
        ctrl->status = (a.epoch << 8) | (fast ? hist::kPathFast : hist::kPathFull);
    }
    if (fast && a.sel_out) {
        // split t's winners go after those of the splits before it
        const uint32_t k = (uint32_t)a.k_blocks;
        const int32_t c = t < ns ? a.stage_n[t] : 0;
        const uint32_t x = wave::incl_scan_add((uint32_t)c);
        if (lane == 63)
            L.wtot[wv] = x;
        __syncthreads();
        uint32_t o = 0;
        for (int w = 0; w < wv; ++w)
            o += L.wtot[w];
        o += x - (uint32_t)c;
        for (int32_t j = 0; j < c; ++j)
            if (o + (uint32_t)j < k)
                a.sel_out[o + j] = a.stage[(size_t)t * k + j];
    }
}

template <int DH, int G>
hipError_t go(const DecodeArgs &a, hipStream_t s)
{
    const size_t lds = sizeof(DecLds<DH, G>);
    if (a.sa.lkeys_off != 0 || sel::lds_bytes(a.sa.nb) > DecLds<DH, G>::kTiles || lds > sel::kMaxLds)
        return hipErrorInvalidConfiguration;
    static hipError_t attr = hipFuncSetAttribute((const void *)k_decode_attend<DH, G>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_decode_attend<DH, G>), dim3(a.ns, a.kv_heads), dim3(kNT), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_decode_merge<DH, G>), dim3(a.kv_heads * G * (DH / kWave) + 1), dim3(kNT), 0, s, a);
    return hipGetLastError();
}

template <int DH>
hipError_t go_g(const DecodeArgs &a, int G, hipStream_t s)
{
    switch (G) {
    case 1: return go<DH, 1>(a, s);
    case 2: return go<DH, 2>(a, s);
    case 4: return go<DH, 4>(a, s);
    case 8: return go<DH, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

namespace {
template <int DH, int G>
bool fits(int64_t nb)
{
    return sizeof(DecLds<DH, G>) <= sel::kMaxLds && nb <= ((int64_t)1 << 19) &&
           sel::lds_bytes((int32_t)nb) <= DecLds<DH, G>::kTiles;
}
template <int DH>
bool fits_g(int64_t nb, int G)
{
    switch (G) {
    case 1: return fits<DH, 1>(nb);
    case 2: return fits<DH, 2>(nb);
    case 4: return fits<DH, 4>(nb);
    case 8: return fits<DH, 8>(nb);
    }
    return false;
}
}  // namespace

bool decode_fits(int64_t nb, int Dh, int G)
{
    switch (Dh) {
    case 64: return fits_g<64>(nb, G);
    case 128: return fits_g<128>(nb, G);
    case 256: return fits_g<256>(nb, G);
    }
    return false;
}

hipError_t launch_decode_attend(const DecodeArgs &a, int Dh, int G, hipStream_t s)
{
    if (a.ns < 1 || a.ns > kDecodeMaxSplits || (int64_t)a.kv_heads * a.ns > kNT ||
        a.n_tail < 0 || a.n_tail > 3 || a.sa.nb > (1 << 19))
        return hipErrorInvalidValue;
    const int64_t per = (a.sa.ntiles + a.ns - 1) / a.ns;
    const int64_t per_k = ((int64_t)a.k_blocks + a.ns - 1) / a.ns;
    if (per * a.sa.T > kNT || per_k > kMaxOwn)
        return hipErrorInvalidValue;
    switch (Dh) {
    case 64: return go_g<64>(a, G, s);
    case 128: return go_g<128>(a, G, s);
    case 256: return go_g<256>(a, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace qsa
