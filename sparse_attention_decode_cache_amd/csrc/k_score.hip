// k_score.hip -- stage 2: stream every cached summary row once and score it.
//
// s[b] = sum_h w[h] * <q_idx[h], summary[b][h]>   [post 10, "QSA indexer"]
//
// This is the only pass whose bytes grow with context (N_b rows of up to 1 KB),
// so it is written as a pure HBM stream.  A row is split over L = min(16,
// LPR) lanes (one DPP row) that each take C = LPR/L of its 16-byte chunks; a
// wave-wide load covers 64/L consecutive rows, L*16 bytes of each: whole
// cache lines, 1 KB per instruction.  Every load of the tile is issued before
// any is used (non-temporal: the rows are not reused in this step).  Each
// lane ends with the partial dots of V rows; a transposing butterfly inside
// the 16-lane row (DPP moves only: row mirror, half mirror, quad swaps)
// finishes V rows in log2(L) rounds.  w[h] is folded into q_idx once per
// workgroup, into LDS.
//
// Outputs (all optional, plain stores): fp32 scores; the order-preserving
// 32-bit key of every score; and, for the top-k, each tile's T largest
// composite keys (key << 32 | ~block), sorted descending (T is chosen per
// call, R/8 .. R/2).  In the decode step every row inside the score window
// also goes into the global score histogram of qsa_hist.h as soon as its
// score is known (before the tile's ranking), by relaxed device-scope
// atomics whose results no lane waits for (count, largest and smallest
// composite of the bin), and the largest last entry of the tiles' lists
// after it; the window is set from the fed-back ratios before the rows
// arrive.
// Up to 4 queries of one sequence (the tokens
// of a speculative-verify call) share one pass: every chunk is loaded once
// and dotted with each query, each query with its own causal block limit.
//
// Fused stage 1: in a decode step at most one summary row is new.  Workgroup 0
// (dispatched first) scores the LAST tile -- the one holding the new row --
// and, while its loads are in flight, appends the token's rows (all of a
// verify call's) and pools that block straight into LDS; the lanes that
// loaded the row's stale chunks take the pooled ones from there.  The
// pooling latency hides under the stream.
#include "qsa_hist.h"
#include "qsa_pool.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

// Lane partner of exchange round O inside a 16-lane row: a lane whose bit O
// differs (mirror moves also flip the lower bits; rounds run from high O to
// low, so lanes differing only in lower bits still hold the same row set).
template <int O>
__device__ inline float partner(float x)
{
    constexpr int ctrl = O == 8 ? wave::kRowMirror
                       : O == 4 ? wave::kRowHalfMirror
                       : O == 2 ? wave::kQuadXor2 : wave::kQuadXor1;
    return __uint_as_float(wave::dpp<ctrl>(__float_as_uint(x)));
}

// Transposing butterfly over the L = 2*O lanes of a row group.  Before:
// v[0..CNT) are partial sums of CNT different rows.  After: v[0] holds the
// full sum of row index `toff` (lanes that end with equal `toff` hold equal
// sums).
template <int O, int CNT>
struct Butterfly {
    static __device__ inline void run(float *v, int lane, int &toff)
    {
        if constexpr (O == 0) {
            return;
        } else if constexpr (CNT > 1) {
            constexpr int H = CNT / 2;
            const bool up = (lane & O) != 0;
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const float send = up ? v[k] : v[k + H];
                const float keep = up ? v[k + H] : v[k];
                v[k] = keep + partner<O>(send);
            }
            if (up)
                toff += H;
            Butterfly<O / 2, H>::run(v, lane, toff);
        } else {
            v[0] += partner<O>(v[0]);
            Butterfly<O / 2, 1>::run(v, lane, toff);
        }
    }
};

// Slot of tile row r in the composites array: with P = 256/R threads
// sharing an entry, each part's span of R/P rows starts 16 bytes further
// along the banks than a plain array would put it, so that the P parts'
// reads in one ranking step fall in distinct banks (unpadded, parts 0 and
// 2 of a 64-row tile read 256 bytes apart: the same banks).
template <int R>
__device__ __forceinline__ int tl_slot(int r)
{
    constexpr int P = 256 / R;
    return P > 1 ? r + 2 * (r / (R / P)) : r;
}
template <int R>
constexpr int tl_size() { return R + 2 * (256 / R); }

// Tile list: the T largest of the R composites in s_c (0 = no row), written
// descending to lists[tile*T ...]; slots past the tile's rows get 0.  T <= R
// is chosen per call (longer lists where a tile holds more winners).  Ranks
// are exact because composites are unique and nonzero.  All 256 threads
// work: P = 256/R consecutive threads share an entry, each counting the
// larger composites in 1/P of the tile, summed with DPP quad moves.  Whole
// workgroup calls (uniform control flow: DPP reads neighbouring lanes).
template <int R>
__device__ inline void write_tile_list(const uint64_t *s_c, uint64_t *lists, int tile, int valid_rows,
                                       int T, const HistOut *h = nullptr, const hist::Map *map = nullptr)
{
    static_assert(R == 64 || R == 128 || R == 256, "tile rows");
    constexpr int P = 256 / R;
    constexpr int SPAN = R / P;
    const int i = threadIdx.x / P, part = threadIdx.x % P;
    const uint64_t c = s_c[tl_slot<R>(i)];
    const uint64_t *span = s_c + tl_slot<R>(part * SPAN);
    uint32_t rank = 0;
#pragma unroll 8
    for (int u = 0; u < SPAN; ++u)
        rank += span[u] > c ? 1u : 0u;
    if constexpr (P >= 2)
        rank += wave::dpp<wave::kQuadXor1>(rank);
    if constexpr (P == 4)
        rank += wave::dpp<wave::kQuadXor2>(rank);
    if (part == 0 && c != 0 && rank < (uint32_t)T) {
        lists[(size_t)tile * T + rank] = c;
        if (h && rank == (uint32_t)T - 1 && valid_rows > T && hist::in_window((uint32_t)(c >> 32), *map))
            // the last entry of a list that may hide rows, inside the window:
            // the maximum of such entries (no result is waited for)
            __hip_atomic_fetch_max(h->last + (tile & (hist::kLast - 1)), c, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    // the nonzero composites take ranks [0, valid_rows): the rest are empty
    if ((int)threadIdx.x >= valid_rows && threadIdx.x < (unsigned)T)
        lists[(size_t)tile * T + threadIdx.x] = 0;
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int LPR>
struct ScoreShape {
    static constexpr int L = LPR < 16 ? LPR : 16;      // lanes per row
    static constexpr int C = LPR / L;                   // chunks per lane per row
    static constexpr int RI = kWave / L;                // rows per wave-wide load
    static constexpr int LOADS = LPR >= 16 ? 16 : 8;    // loads per lane
    static constexpr int V = LOADS / C;                 // row groups per lane
    static constexpr int RPW = V * RI;                  // rows per wave
    static constexpr int R = 4 * RPW;                   // rows per workgroup tile
    static_assert(V >= 1 && V <= L, "one butterfly finishes the rows");
};

// One tile for Q queries of one sequence (Q = 1: the decode step; Q > 1:
// speculative verify of consecutive tokens): the tile's rows are loaded
// once and every 16-byte chunk is widened once and dotted with all Q
// queries.  The folded queries w[h] q[h] sit in LDS and are read one chunk
// position at a time, so the registers hold the row loads, one chunk of
// every query and Q x V sums whatever Q is (122 VGPRs for 1 KB rows: four
// workgroups per CU, so a 256k-context grid of ~1000 tiles is resident at
// once).  Query i sees the rows below a.nbq[i]; the rest get no key, no
// list entry and a score of -inf.  The butterfly, keys and lists run once
// per query.
// Slot (in float4s) of quarter k4 of row chunk ch in the folded queries:
// the H = EPL/4 float4s of a chunk are stored apart, L chunks to a run, so
// that the L lanes of a row reading quarter k4 of chunks ch0 .. ch0+L-1 read
// L consecutive float4s (no two in the same banks).  The squared-norm sum
// of the histogram window reads every element and does not depend on the
// order.
template <int L, int H>
__device__ __forceinline__ int q_slot(int ch, int k4)
{
    return (ch / L) * (H * L) + k4 * L + ch % L;
}

template <int LPR, int Q, int EPL>
struct ScoreMultiLds {
    float qw[Q][LPR * EPL];
    uint64_t c[Q][tl_size<ScoreShape<LPR>::R>()];
    u32x4 fresh[LPR];
    float gam[128];             // RMSNorm weights (histogram window)
};

template <bool F16, int LPR, int Q>
using ScoreLdsOf = ScoreMultiLds<LPR, Q, F16 ? 8 : 4>;

// Score tile `tile` for Q queries (256 threads).  `pool_here`: this
// workgroup runs the fused append + pool (it must hold the last tile).
template <bool F16, int LPR, int Q>
__device__ inline void score_tile(const ScoreMultiArgs &a, ScoreLdsOf<F16, LPR, Q> &sl, int tile,
                                  bool pool_here)
{
    using S = ScoreShape<LPR>;
    constexpr int EPL = F16 ? 8 : 4;
    constexpr int L = S::L, C = S::C, RI = S::RI, V = S::V, R = S::R;
    constexpr int ROWB = LPR * 16;
    constexpr int HD = LPR * EPL;              // elements of a row
    constexpr int QPT = (Q * HD / 4 + 255) / 256;   // float4 groups of queries per thread

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane % L;
    const int sub = lane / L;
    const int64_t base = (int64_t)tile * R + (int64_t)wave * S::RPW;

    // the fed-back histogram window and gamma (for its scale), loaded with
    // the queries ahead of the rows so that the window is set while the rows
    // are in flight
    float rho_k = 0.0f, rho_top = 0.0f;
    if (Q == 1 && a.h.hist) {
        const hist::Ctrl *ctrl = reinterpret_cast<const hist::Ctrl *>(a.h.ctrl);
        const bool fed = ctrl->fb == hist::kFeedback;
        rho_k = fed ? ctrl->rho_k : __builtin_nanf("");   // NaN: the default window
        rho_top = ctrl->rho_top;
    }
    // gamma entry t (thread t < D), staged through LDS like the queries: the
    // load is unconditional (any readable word without a window) so that
    // nothing waits for it before the rows are issued
    const bool want_g = Q == 1 && a.h.hist != nullptr;
    const float *gsrc = want_g ? a.h.gamma : a.w[0];
    const float graw = gsrc[want_g && (int)threadIdx.x < a.D ? (int)threadIdx.x : 0];
    // the queries' float4 groups this thread folds into LDS, loaded ahead of the rows
    float4 qraw[QPT];
    float wraw[QPT];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int g4 = (int)threadIdx.x + 256 * j;
        if (g4 < Q * HD / 4) {
            const int qi = g4 / (HD / 4), e0 = 4 * (g4 % (HD / 4));
            qraw[j] = ((const float4 *)(a.q[qi] + e0))[0];
            wraw[j] = a.w[qi][e0 / a.D];
        }
    }
    // The pool of a completed block runs before this tile's rows are
    // requested: loads are counted in issue order, so pool loads issued after
    // the rows would wait for the whole tile, and the pool's double-precision
    // chain would then start only when the tile is in, which can be the end
    // of the pass.  The pooled row reaches this tile through LDS.
    // The appended token's rows are fetched ahead of the tile for the same
    // reason, and stored once the tile's loads are out.
    const bool app = pool_here && a.upd.new_idx_row;
    AppendWords aw;
    if (app)
        append_fetch(a.upd, threadIdx.x, 256, aw);
    if (pool_here && a.upd.nblk > 0)
        pool_row<F16>(a.upd, a.upd.b0, threadIdx.x, sl.fresh);
    __builtin_amdgcn_sched_barrier(0);

    const char *rows = (const char *)a.summary;
    u32x4 buf[S::LOADS];
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
        const int64_t r = base + (int64_t)(i / C) * RI + sub;
        const u32x4 *src = (const u32x4 *)(rows + (r < a.nb ? r : 0) * ROWB) + col + L * (i % C);
        buf[i] = __builtin_nontemporal_load(src);
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int g4 = (int)threadIdx.x + 256 * j;
        if (g4 < Q * HD / 4) {
            const int qi = g4 / (HD / 4), e0 = 4 * (g4 % (HD / 4));
            float4 f = qraw[j];
            f.x *= wraw[j];
            f.y *= wraw[j];
            f.z *= wraw[j];
            f.w *= wraw[j];
            *(float4 *)&sl.qw[qi][4 * q_slot<L, EPL / 4>(e0 / EPL, (e0 % EPL) / 4)] = f;
        }
    }

    if (want_g && (int)threadIdx.x < a.D)
        sl.gam[threadIdx.x] = graw;

    if (app)
        append_put(a.upd, threadIdx.x, 256, aw);
    __syncthreads();
    if (pool_here && a.upd.nblk > 0) {
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int64_t r = base + (int64_t)(i / C) * RI + sub;
            if (r == a.upd.b0)
                buf[i] = sl.fresh[col + L * (i % C)];
        }
    }
    hist::Map map{};
    if (Q == 1 && a.h.hist) {
        // the histogram window (qsa_hist.h), every wave alike: its scale from
        // the folded query's squared norm and the mean of gamma^2
        float ss = 0.0f, gg = 0.0f;
#pragma unroll
        for (int j = 0; j < HD / kWave; ++j) {
            const float x = sl.qw[0][lane + kWave * j];
            ss = fmaf(x, x, ss);
        }
        for (int e = lane; e < a.D; e += kWave)
            gg = fmaf(sl.gam[e], sl.gam[e], gg);
        ss = wave::reduce_add_f(ss);
        gg = wave::reduce_add_f(gg);
        const float sigma = sqrtf(ss * (gg / (float)a.D));
        float lo, mid, hi;
        hist::window(sigma, rho_k, rho_top, a.h.def_k, a.h.def_top, lo, mid, hi);
        map = hist::make_map(lo, mid, hi);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            // stamp the region with this call (clean start or not) and leave the
            // window and its bin map for the attention kernel
            hist::Ctrl *ctrl = reinterpret_cast<hist::Ctrl *>(a.h.ctrl);
            ctrl->tag = ctrl->tag == hist::kTagClean ? hist::tag_ok(a.h.epoch) : hist::tag_bad(a.h.epoch);
            ctrl->sigma = sigma;
            ctrl->lo = lo;
            ctrl->mid = mid;
            ctrl->hi = hi;
            ctrl->inv1 = map.inv1;
            ctrl->inv2 = map.inv2;
            ctrl->klo = map.klo;
            ctrl->kmid = map.kmid;
            ctrl->khi = map.khi;
            ctrl->map_ok = map.ok ? 1u : 0u;
        }
    }
    float v[Q][V];
#pragma unroll
    for (int qi = 0; qi < Q; ++qi)
#pragma unroll
        for (int g = 0; g < V; ++g)
            v[qi][g] = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        float qw[Q][EPL];
#pragma unroll
        for (int qi = 0; qi < Q; ++qi)
#pragma unroll
            for (int k4 = 0; k4 < EPL / 4; ++k4) {
                const float4 f = *(const float4 *)&sl.qw[qi][4 * q_slot<L, EPL / 4>(col + L * c, k4)];
                qw[qi][4 * k4] = f.x;
                qw[qi][4 * k4 + 1] = f.y;
                qw[qi][4 * k4 + 2] = f.z;
                qw[qi][4 * k4 + 3] = f.w;
            }
#pragma unroll
        for (int g = 0; g < V; ++g) {
            const u32x4 &b = buf[g * C + c];
            if constexpr (F16) {
                half8 h;
                __builtin_memcpy(&h, &b, 16);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float x = (float)h[k];
#pragma unroll
                    for (int qi = 0; qi < Q; ++qi)
                        v[qi][g] = fmaf(qw[qi][k], x, v[qi][g]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float x = __uint_as_float(b[k]);
#pragma unroll
                    for (int qi = 0; qi < Q; ++qi)
                        v[qi][g] = fmaf(qw[qi][k], x, v[qi][g]);
                }
            }
        }
    }

    int toff = 0;
#pragma unroll
    for (int qi = 0; qi < Q; ++qi) {
        int t = 0;
        Butterfly<L / 2, V>::run(v[qi], lane, t);
        toff = t;                              // the same for every query
    }

    constexpr int OWN = L / V;
    const int local = wave * S::RPW + toff * RI + sub;
    const int64_t r = (int64_t)tile * R + local;
    if (col % OWN == 0) {
#pragma unroll
        for (int qi = 0; qi < Q; ++qi) {
            uint64_t c = 0;
            if (r < a.nbq[qi]) {
                const float sc = v[qi][0];
                if (a.scores)
                    a.scores[qi * a.ld_scores + r] = sc;
                if (a.keys[qi]) {
                    const uint32_t key = score_key(sc);
                    a.keys[qi][r] = key;
                    c = comp_key(key, (uint32_t)r);
                    if (Q == 1 && a.h.hist && map.ok && hist::in_window(key, map)) {
                        // every row inside the window goes into its bin now,
                        // before the tile's ranking (the counts are then of
                        // all rows >= L, not only listed ones: exact)
                        const uint32_t b = hist::bin_of(key, map);
                        __hip_atomic_fetch_add(a.h.hist + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_fetch_max(a.h.bmax + b, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_fetch_max(a.h.bminc + b, ~c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            } else if (r < a.nb && a.scores) {
                a.scores[qi * a.ld_scores + r] = -__builtin_inff();
            }
            sl.c[qi][tl_slot<R>(local)] = c;
        }
    }
    __syncthreads();
    if (Q == 1 && a.h.hist) {
        const int64_t valid = a.nbq[0] - (int64_t)tile * R;
        write_tile_list<R>(sl.c[0], a.lists[0], tile, (int)(valid < 0 ? 0 : (valid < R ? valid : R)),
                           a.list_t, map.ok ? &a.h : nullptr, &map);
        return;
    }
#pragma unroll
    for (int qi = 0; qi < Q; ++qi) {
        if (a.lists[qi]) {
            const int64_t valid = a.nbq[qi] - (int64_t)tile * R;
            write_tile_list<R>(sl.c[qi], a.lists[qi], tile,
                               (int)(valid < 0 ? 0 : (valid < R ? valid : R)), a.list_t);
        }
    }
}

template <bool F16, int LPR, int Q>
__global__ __launch_bounds__(256) void k_score_multi(ScoreMultiArgs a)
{
    __shared__ ScoreLdsOf<F16, LPR, Q> sl;
    // workgroup 0 (dispatched first) takes the last tile: the one holding the new row
    const int tile = blockIdx.x == 0 ? (int)gridDim.x - 1 : (int)blockIdx.x - 1;
    score_tile<F16, LPR, Q>(a, sl, tile, blockIdx.x == 0 && a.fuse);
}

// One query: the same tile routine.
__device__ inline ScoreMultiArgs single(const ScoreArgs &a)
{
    ScoreMultiArgs m{};
    m.summary = a.summary;
    m.nb = a.nb;
    m.D = a.D;
    m.fuse = a.fuse;
    m.upd = a.upd;
    m.nbq[0] = a.nb;
    m.q[0] = a.q;
    m.w[0] = a.w;
    m.keys[0] = a.keys;
    m.lists[0] = a.lists;
    m.scores = a.scores;
    m.ld_scores = 0;
    m.list_t = a.list_t;
    m.h = a.h;
    return m;
}

template <bool F16, int LPR>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a)
{
    __shared__ ScoreLdsOf<F16, LPR, 1> sl;
    const int tile = blockIdx.x == 0 ? (int)gridDim.x - 1 : (int)blockIdx.x - 1;
    score_tile<F16, LPR, 1>(single(a), sl, tile, blockIdx.x == 0 && a.fuse);
}

// A batch of sequences in one launch: workgroups [tile0[s], tile0[s+1]) score
// sequence s, the first of them its last tile (with the fused prologue).
template <bool F16, int LPR>
__global__ __launch_bounds__(256) void k_score_batch(ScoreBatchArgs b)
{
    __shared__ ScoreLdsOf<F16, LPR, 1> sl;
    int s = 0;
    while (s + 1 < b.n && (int)blockIdx.x >= b.tile0[s + 1])
        ++s;
    const int local = (int)blockIdx.x - b.tile0[s];
    const int ntiles = b.tile0[s + 1] - b.tile0[s];
    const int tile = local == 0 ? ntiles - 1 : local - 1;
    score_tile<F16, LPR, 1>(single(b.seq[s]), sl, tile, local == 0 && b.seq[s].fuse);
}

template <bool F16, int LPR>
hipError_t go_multi(const ScoreMultiArgs &a, int n_q, hipStream_t s)
{
    const int grid = (int)((a.nb + ScoreShape<LPR>::R - 1) / ScoreShape<LPR>::R);
    switch (n_q) {
    case 1: hipLaunchKernelGGL((k_score_multi<F16, LPR, 1>), dim3(grid), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_score_multi<F16, LPR, 2>), dim3(grid), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_score_multi<F16, LPR, 3>), dim3(grid), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_score_multi<F16, LPR, 4>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Keys and tile lists from given fp32 scores (stand-alone top-k), R = 256.
__global__ __launch_bounds__(kKeysTile) void k_keys(const float *scores, int32_t nb, uint32_t *keys,
                                                    uint64_t *lists)
{
    __shared__ uint64_t s_c[kKeysTile];
    const int i = blockIdx.x * kKeysTile + threadIdx.x;
    uint64_t c = 0;
    if (i < nb) {
        const uint32_t key = score_key(scores[i]);
        keys[i] = key;
        c = comp_key(key, (uint32_t)i);
    }
    s_c[threadIdx.x] = c;
    __syncthreads();
    const int valid = nb - (int)blockIdx.x * kKeysTile;
    write_tile_list<kKeysTile>(s_c, lists, blockIdx.x, valid < kKeysTile ? valid : kKeysTile,
                               kKeysTile / kListDiv);
}

template <bool F16, int LPR>
hipError_t go(const ScoreArgs &a, hipStream_t s)
{
    const int grid = (int)((a.nb + ScoreShape<LPR>::R - 1) / ScoreShape<LPR>::R);
    hipLaunchKernelGGL((k_score<F16, LPR>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int score_tile_rows(bool f16, int row_bytes)
{
    switch (row_bytes / 16) {
    case 8: return f16 ? ScoreShape<8>::R : 0;
    case 16: return ScoreShape<16>::R;
    case 32: return ScoreShape<32>::R;
    case 64: return ScoreShape<64>::R;
    }
    return 0;
}

hipError_t launch_score(const ScoreArgs &a, bool f16, int row_bytes, hipStream_t s)
{
    if (a.nb <= 0)
        return hipSuccess;
    const int lpr = row_bytes / 16;
    if (f16) {
        switch (lpr) {
        case 8: return go<true, 8>(a, s);
        case 16: return go<true, 16>(a, s);
        case 32: return go<true, 32>(a, s);
        case 64: return go<true, 64>(a, s);
        }
    } else {
        switch (lpr) {
        case 16: return go<false, 16>(a, s);
        case 32: return go<false, 32>(a, s);
        case 64: return go<false, 64>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_score_batch(ScoreBatchArgs &b, bool f16, int row_bytes, hipStream_t s)
{
    const int R = score_tile_rows(f16, row_bytes);
    if (R == 0 || b.n < 1 || b.n > kMaxBatch)
        return hipErrorInvalidValue;
    b.tile0[0] = 0;
    for (int i = 0; i < b.n; ++i) {
        const int nt = (int)((b.seq[i].nb + R - 1) / R);
        b.tile0[i + 1] = b.tile0[i] + (nt > 0 ? nt : 1);   // at least one: the fused prologue
    }
    const int grid = b.tile0[b.n];
    const int lpr = row_bytes / 16;
    if (f16) {
        switch (lpr) {
        case 8: hipLaunchKernelGGL((k_score_batch<true, 8>), dim3(grid), dim3(256), 0, s, b); break;
        case 16: hipLaunchKernelGGL((k_score_batch<true, 16>), dim3(grid), dim3(256), 0, s, b); break;
        case 32: hipLaunchKernelGGL((k_score_batch<true, 32>), dim3(grid), dim3(256), 0, s, b); break;
        case 64: hipLaunchKernelGGL((k_score_batch<true, 64>), dim3(grid), dim3(256), 0, s, b); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (lpr) {
        case 16: hipLaunchKernelGGL((k_score_batch<false, 16>), dim3(grid), dim3(256), 0, s, b); break;
        case 32: hipLaunchKernelGGL((k_score_batch<false, 32>), dim3(grid), dim3(256), 0, s, b); break;
        case 64: hipLaunchKernelGGL((k_score_batch<false, 64>), dim3(grid), dim3(256), 0, s, b); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_score_multi(const ScoreMultiArgs &a, int n_q, bool f16, int row_bytes,
                              hipStream_t s)
{
    if (a.nb <= 0)
        return hipSuccess;
    const int lpr = row_bytes / 16;
    if (f16) {
        switch (lpr) {
        case 8: return go_multi<true, 8>(a, n_q, s);
        case 16: return go_multi<true, 16>(a, n_q, s);
        case 32: return go_multi<true, 32>(a, n_q, s);
        case 64: return go_multi<true, 64>(a, n_q, s);
        }
    } else {
        switch (lpr) {
        case 16: return go_multi<false, 16>(a, n_q, s);
        case 32: return go_multi<false, 32>(a, n_q, s);
        case 64: return go_multi<false, 64>(a, n_q, s);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_keys(const float *scores, int32_t nb, uint32_t *keys, uint64_t *lists,
                       hipStream_t s)
{
    if (nb <= 0)
        return hipSuccess;
    const int grid = (nb + kKeysTile - 1) / kKeysTile;
    hipLaunchKernelGGL(k_keys, dim3(grid), dim3(kKeysTile), 0, s, scores, nb, keys, lists);
    return hipGetLastError();
}

}  // namespace qsa
