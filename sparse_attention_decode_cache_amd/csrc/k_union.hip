// k_union.hip -- grouped-union attention of a prefill chunk (a reading of
// post 10's "QSA grouped-union", which sped up prefill and is not defined on
// the page; its opening paragraphs, "Vulkan版のプロファイリングでTGが遅くなった
// 原因を調べる" and the prefill paragraph of "COMMON-004実装結果" name it).
//
// Reading: consecutive queries of the chunk form groups; a group reads the
// K / V rows of the union of its queries' chosen blocks (and of its queries'
// tail cells) once, and each query attends over that union with every cell
// that is not its own masked out, so each query's output is its own QSA
// attention (the same cells as the per-query path).
//
// A group is as many queries as fill 64 query x head rows, four 16-row
// matrix-core tiles: QG = 64 / G queries of G heads each (at most 32, the
// bits of a union block's mask; fewer when their bitmaps would not fit the
// build's LDS), so that every K / V row read serves up to QG queries.
//   build   one workgroup per group: the queries' ids as bitmaps in LDS, OR-ed
//           and compacted in ascending order into the group's union list,
//           with each union block's mask of the queries that chose it;
//   attend  workgroup (group, KV head), 512 threads: the union's cells (4 per
//           block, ascending) and then the group's tail range [4 floor(n_first
//           / 4), n_last), 64 cells per iteration: K and V rows land in an LDS
//           tile once for the whole group (their loads one iteration ahead,
//           the union ids they need two ahead, read from memory); the logits
//           of all QG x G rows on the matrix cores (q as f16 hi + lo; a wave
//           per 16 cells and up to two row tiles), a cell counting for a row
//           only if it is that query's own (the block's mask, loaded an
//           iteration ahead); online softmax per row; P.V on the matrix cores
//           (a wave per 16-dim slice, its V operand shared by the row tiles);
//           the output written normalised per query.
#include "qsa_internal.h"
#include "qsa_unit.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

constexpr int kUB = 512;                     // build threads
constexpr int kUT = 512;                     // attend threads
constexpr int kUW = kUT / kWave;
constexpr int kUC = 64;                      // cells per iteration
constexpr int kMaxRT = kUnionMaxRows / 16;  // 16-row matrix-core tiles of a group

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Block ids of query i of the chunk (ascending): its chosen ones, or all of
// its completed blocks when it keeps them all.
__device__ inline int32_t query_nb(const ChunkArgs &c, int i) { return (c.n0 + i + 1) / 4; }

__global__ __launch_bounds__(kUB) void k_union_build(ChunkArgs c)
{
    extern __shared__ uint32_t ub_lds[];
    const int QG = c.union_q;
    const int j = blockIdx.x, q0 = j * QG;
    const int nqg = c.n_q - q0 < QG ? c.n_q - q0 : QG;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int32_t nb_hi = query_nb(c, q0 + nqg - 1);
    const int W = (nb_hi + 31) / 32;
    uint32_t *bm = ub_lds;                         // [QG][W]
    uint32_t *wtot = ub_lds + (size_t)QG * W;      // [kUB / 64]
    for (int x = t; x < QG * W; x += kUB)
        bm[x] = 0u;
    __syncthreads();
    for (int qi = 0; qi < nqg; ++qi) {
        const int i = q0 + qi;
        const int32_t nbi = query_nb(c, i);
        const bool all = nbi <= c.kb;
        const int32_t ki = all ? nbi : c.kb;
        const int32_t *row = c.sel + (size_t)i * c.kb;
        for (int32_t x = t; x < ki; x += kUB) {
            const int32_t id = all ? x : row[x];
            atomicOr(&bm[(size_t)qi * W + (id >> 5)], 1u << (id & 31));
        }
    }
    __syncthreads();
    // thread t: words [t per, (t + 1) per); counts, then an exclusive scan
    const int per = (W + kUB - 1) / kUB;
    const int w0 = t * per, w1 = w0 + per < W ? w0 + per : W;
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) {
        uint32_t u = 0;
        for (int qi = 0; qi < nqg; ++qi)
            u |= bm[(size_t)qi * W + w];
        cnt += (uint32_t)__popc(u);
    }
    const uint32_t incl = wave::incl_scan_add(cnt);
    if (lane == 63)
        wtot[wv] = incl;
    __syncthreads();
    uint32_t pos = incl - cnt;
    for (int w = 0; w < wv; ++w)
        pos += wtot[w];
    int32_t *uni = c.uni + (size_t)j * c.ucap;
    uint32_t *msk = c.umask + (size_t)j * c.ucap;
    for (int w = w0; w < w1; ++w) {
        uint32_t u = 0;
        for (int qi = 0; qi < nqg; ++qi)
            u |= bm[(size_t)qi * W + w];
        while (u) {
            const int b = __ffs(u) - 1;
            u &= u - 1u;
            uint32_t m = 0;
            for (int qi = 0; qi < nqg; ++qi)
                m |= ((bm[(size_t)qi * W + w] >> b) & 1u) << qi;
            uni[pos] = 32 * w + b;
            msk[pos] = m;
            ++pos;
        }
    }
    if (t == kUB - 1)
        c.ucount[j] = (int32_t)pos;
}

// Max / sum over aligned groups of N consecutive lanes (N = 8, 16 or 32);
// every lane of a group ends with its group's result.
template <int N>
__device__ inline float group_max(float v)
{
    static_assert(N == 8 || N == 16 || N == 32, "groups of 8, 16 or 32 lanes");
    auto mx = [](float a, uint32_t b) { return fmaxf(a, __uint_as_float(b)); };
    v = mx(v, wave::dpp<wave::kQuadXor1>(__float_as_uint(v)));
    v = mx(v, wave::dpp<wave::kQuadXor2>(__float_as_uint(v)));
    v = mx(v, wave::dpp<wave::kRowHalfMirror>(__float_as_uint(v)));
    if constexpr (N >= 16)
        v = mx(v, wave::dpp<wave::kRowMirror>(__float_as_uint(v)));
    if constexpr (N == 32)
        v = fmaxf(v, __shfl_xor(v, 16));
    return v;
}

template <int N>
__device__ inline float group_sum(float v)
{
    static_assert(N == 8 || N == 16 || N == 32, "groups of 8, 16 or 32 lanes");
    auto ad = [](float a, uint32_t b) { return a + __uint_as_float(b); };
    v = ad(v, wave::dpp<wave::kQuadXor1>(__float_as_uint(v)));
    v = ad(v, wave::dpp<wave::kQuadXor2>(__float_as_uint(v)));
    v = ad(v, wave::dpp<wave::kRowHalfMirror>(__float_as_uint(v)));
    if constexpr (N >= 16)
        v = ad(v, wave::dpp<wave::kRowMirror>(__float_as_uint(v)));
    if constexpr (N == 32)
        v += __shfl_xor(v, 16);
    return v;
}

template <int DH, int RT>
struct UShape {
    static constexpr int KS = DH / 32;              // MFMA k-steps of a row
    static constexpr int KROW = 2 * DH + 16;        // padded LDS bytes of a K row
    static constexpr int VROW = DH >= 128 ? 2 * DH + 32 : KROW;   // and of a V row (unit::vswz)
    static constexpr int CH = DH / 8;               // 16-byte chunks of a row
    static constexpr int PAIRS = kUC * CH;          // (cell, chunk) pairs of an iteration
    static constexpr int PR = PAIRS / kUT;
    static_assert(PAIRS % kUT == 0 && PR <= 8, "whole (cell, chunk) pairs per thread, at most 8");
    static constexpr int RW = 16 * RT;              // rows of the group's tiles
    static constexpr int TPR = kUT / RW;            // softmax threads per row (8, 16, 32)
    static constexpr int CPS = kUC / TPR;           // cells per softmax thread (8, 4, 2)
    static constexpr int LGS = kUC + 4;             // floats per logit row (16-byte aligned, padded)
    static constexpr int LW = RT == 1 ? 4 : 8;      // waves taking logits (one 16-cell tile each)
    static constexpr int LRT = 4 * RT / LW;         // row tiles per logit wave
    static constexpr int NT = DH / 16;              // 16-dim output tiles
    static constexpr int TPW = (NT + kUW - 1) / kUW;
    static_assert(RT == 1 || RT == 2 || RT == kMaxRT, "one, two or four row tiles");
};

template <int DH, int RT>
struct ULds {
    using S = UShape<DH, RT>;
    alignas(16) unsigned char ktile[kUC * (S::VROW > S::KROW ? S::VROW : S::KROW)];   // K, then V, of the iteration
    alignas(16) uint4 qb[RT][S::KS][2][kWave];
    alignas(16) float lg[S::RW][S::LGS];
    alignas(16) _Float16 pt[2][S::RW][kUC + 8];     // rows padded: a P.V read's rows 4 banks apart
    float sc[S::RW], lrow[S::RW];
};

template <int DH, int G, int RT>
__global__ __launch_bounds__(kUT) void k_union_attend(ChunkArgs c)
{
    using S = UShape<DH, RT>;
    constexpr int KS = S::KS, KROW = S::KROW, VROW = S::VROW, CH = S::CH, PR = S::PR, TPR = S::TPR, CPS = S::CPS,
                  LW = S::LW, LRT = S::LRT, NT = S::NT, TPW = S::TPW;
    extern __shared__ uint4 ua_lds[];
    ULds<DH, RT> &L = *reinterpret_cast<ULds<DH, RT> *>(ua_lds);
    const int QG = c.union_q;
    const int R = QG * G;                          // rows in use (<= RW)
    const int j = blockIdx.x, g = blockIdx.y, q0 = j * QG;
    const int nqg = c.n_q - q0 < QG ? c.n_q - q0 : QG;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int32_t nu = c.ucount[j];
    const int64_t n_first = (int64_t)c.n0 + q0 + 1, n_last = (int64_t)c.n0 + q0 + nqg;
    const int64_t t0 = n_first / 4 * 4;
    const int32_t ncells = 4 * nu + (int32_t)(n_last - t0);
    const int32_t nit = (ncells + kUC - 1) / kUC;
    const int32_t *uni = c.uni + (size_t)j * c.ucap;
    const uint32_t *umsk = c.umask + (size_t)j * c.ucap;
    // q of the group's rows (row r: query r / G, head g G + r % G) as the
    // logit MFMA's B operand: tile rt, k-step ks, lane l holds row 16 rt + l
    // % 16, dims 32 ks + 8 (l / 16) .. +8, zero past the rows in use
    for (int x = t; x < RT * KS * kWave; x += kUT) {
        const int rt = x / (KS * kWave), ks = x / kWave % KS, l = x % kWave;
        const int r = 16 * rt + l % 16, d0 = 32 * ks + 8 * (l / 16);
        const int qi = r / G, h = r % G;
        float4 u = make_float4(0.0f, 0.0f, 0.0f, 0.0f), v = u;
        if (r < R && qi < nqg) {
            const float *qp = c.q + ((size_t)(q0 + qi) * c.kv_heads * G + (size_t)g * G + h) * DH + d0;
            u = *(const float4 *)qp;
            v = *(const float4 *)(qp + 4);
        }
        const float qf[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        half8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = (_Float16)qf[e];
            lo[e] = (_Float16)(qf[e] - (float)hi[e]);
        }
        __builtin_memcpy(&L.qb[rt][ks][0][l], &hi, 16);
        __builtin_memcpy(&L.qb[rt][ks][1][l], &lo, 16);
    }

    // K and V one iteration ahead and the union ids two ahead, in registers
    // named at compile time (an array indexed across the iteration loop ends
    // up in scratch memory): thread t takes the (cell, chunk) pairs t + 512 r.
    // The lambdas see copies of the kernel arguments they use (taking the
    // address of the argument block would copy it to scratch memory).
    const uint16_t *kp = c.k, *vp = c.v;
    const int kvh = c.kv_heads;
    auto load_ids = [=](int it, unit::Regs8<int32_t> &id) __attribute__((always_inline)) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int32_t eb = (kUC * it + (t + kUT * r) / CH) >> 2;
            const int32_t v = uni[eb < nu ? eb : 0];
            id.template at<r>() = eb < nu ? v : 0;
        });
    };
    auto row_base = [=](int it, int pr, int32_t id) __attribute__((always_inline)) -> size_t {
        const int32_t e = kUC * it + pr / CH;
        int64_t cell = 0;
        if (e < ncells)
            cell = e < 4 * nu ? 4 * (int64_t)id + (e & 3) : t0 + (e - 4 * nu);
        return ((size_t)cell * kvh + g) * DH + 8 * (pr % CH);
    };
    auto load_rows = [=](const uint16_t *src, int it, unit::Regs8<int32_t> &id, unit::Regs8<u32x4> &rr)
        __attribute__((always_inline)) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            rr.template at<r>() = *(const u32x4 *)(src + row_base(it, t + kUT * r, id.template at<r>()));
        });
    };
    // the logit waves: wave w takes cells 16 (w % 4) .. +16 of an iteration
    // and row tiles (w / 4) LRT .. +LRT; lane l the union block of cells
    // 16 (w % 4) + 4 (l / 16) .. +4, whose query mask it loads an iteration
    // ahead
    const int ct = wave & 3, rt0 = (wave >> 2) * LRT;
    const int mc = lane & 15, kg = lane >> 4;
    auto load_mask = [=](int it) __attribute__((always_inline)) -> uint32_t {
        const int32_t eb = 16 * it + 4 * ct + kg;
        const uint32_t v = umsk[eb < nu ? eb : 0];
        return eb < nu ? v : 0u;
    };
    // per logit row of the lane (16 (rt0 + i) + mc): its query's bit (0 for
    // rows past the group's) and its tail cells [tlo, thi) counted from t0
    uint32_t qbit[LRT];
    int32_t tlo[LRT], thi[LRT];
#pragma unroll
    for (int i = 0; i < LRT; ++i) {
        const int r = 16 * (rt0 + i) + mc, qi = r / G;
        const bool live = r < R && qi < nqg;
        qbit[i] = live ? 1u << qi : 0u;
        tlo[i] = live ? (int32_t)((n_first + qi) / 4 * 4 - t0) : 0;
        thi[i] = live ? (int32_t)(n_first + qi - t0) : 0;
    }
    const int hn = lane & 15, kq = lane >> 4;
    float4v acc[TPW][RT];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            acc[i][rt] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    // the softmax: TPR consecutive threads per row, CPS cells each
    const int sr = t / TPR, sc0 = CPS * (t % TPR);
    float m_run = -INFINITY, l_run = 0.0f;
    // K and V one iteration ahead, the union ids two ahead in two register
    // sets that trade roles every iteration (so the loop runs two iterations
    // per trip: copying a set whose loads are in flight would wait for
    // them).  Every load is issued unconditionally (past the last iteration,
    // or past the union, from a valid dummy address): a load skipped on some
    // path makes the compiler's wait counts assume the fewest loads in
    // flight, and a store of this iteration's rows would then wait for the
    // rows of the next.
    const float scale = c.scale;
    unit::Regs8<u32x4> kc, vc;
    unit::Regs8<int32_t> i0, i1;
    load_ids(0, i0);
    load_rows(kp, 0, i0, kc);
    load_rows(vp, 0, i0, vc);
    load_ids(1, i1);
    uint32_t mreg = load_mask(0);
    __syncthreads();                                                    // barrier: q operand
    // iteration it: kc / vc hold its K / V rows (and then take those of it +
    // 1), ia the ids of it + 1, ib takes those of it + 2
    auto step = [&](int32_t it, unit::Regs8<int32_t> &ia, unit::Regs8<int32_t> &ib) __attribute__((always_inline)) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + kUT * r;
            *(u32x4 *)(L.ktile + (pr / CH) * KROW + 16 * ((pr % CH) ^ unit::swz(pr / CH))) = kc.template at<r>();
        });
        load_ids(it + 2, ib);
        load_rows(kp, it + 1, ia, kc);
        __syncthreads();                                                // barrier: K tile
        if (wave < LW) {
            // D[cell][row] = K[cell][:] . q[row][:]
            float4v d[LRT], ee[LRT];
#pragma unroll
            for (int i = 0; i < LRT; ++i) {
                d[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
                ee[i] = d[i];
            }
            // operands of k-step ks + 1 read while those of ks feed the
            // matrix cores (two register sets, by k-step parity)
            half8 a[2], bh[2][LRT], bl[2][LRT];
            auto fetch = [&](int ks, int b) __attribute__((always_inline)) {
                __builtin_memcpy(&a[b], L.ktile + (16 * ct + mc) * KROW + 16 * ((4 * ks + kg) ^ unit::swz(16 * ct + mc)), 16);
#pragma unroll
                for (int i = 0; i < LRT; ++i) {
                    __builtin_memcpy(&bh[b][i], &L.qb[rt0 + i][ks][0][lane], 16);
                    __builtin_memcpy(&bl[b][i], &L.qb[rt0 + i][ks][1][lane], 16);
                }
            };
            fetch(0, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int b = ks & 1;
                if (ks + 1 < KS)
                    fetch(ks + 1, b ^ 1);
#pragma unroll
                for (int i = 0; i < LRT; ++i) {
                    d[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b], bh[b][i], d[i], 0, 0, 0);
                    ee[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b], bl[b][i], ee[i], 0, 0, 0);
                }
            }
            // the lane's 4 cells: one union block (its query mask), or tail
            // cells (each query's own range) and cells past the last
            // (bitwise tests, no short-circuit: no branch per element)
            const int32_t e0 = kUC * it + 16 * ct + 4 * kg;
            const bool inu = e0 < 4 * nu;
#pragma unroll
            for (int i = 0; i < LRT; ++i) {
                const bool uo = (mreg & qbit[i]) != 0u;
                float4v v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int32_t x = e0 + q - 4 * nu;
                    const bool to = (e0 + q < ncells) & (x >= tlo[i]) & (x < thi[i]);
                    v[q] = (inu ? uo : to) ? scale * (d[i][q] + ee[i][q]) : -INFINITY;
                }
                *(float4v *)&L.lg[16 * (rt0 + i) + mc][16 * ct + 4 * kg] = v;
            }
        }
        mreg = load_mask(it + 1);
        __syncthreads();                                                // barrier: logits
        // online softmax: row sr, cells sc0 .. +CPS of this thread (rows are
        // whole aligned groups of TPR lanes, so the group reductions stay
        // among live lanes)
        if (sr < R) {
            float x[CPS];
            __builtin_memcpy(x, &L.lg[sr][sc0], sizeof(x));
            float mx = x[0];
#pragma unroll
            for (int e = 1; e < CPS; ++e)
                mx = fmaxf(mx, x[e]);
            // (a row with no cell yet keeps m = -inf: its weights and the
            // rescale of its zero sums are exp(-inf) = 0, taken against 0)
            const float mn = fmaxf(m_run, group_max<TPR>(mx));
            const float ms = mn == -INFINITY ? 0.0f : mn;
            const float scl = expf(m_run - ms);
            float p[CPS], ps = 0.0f;
#pragma unroll
            for (int e = 0; e < CPS; ++e) {
                p[e] = expf(x[e] - ms);
                ps += p[e];
            }
            l_run = l_run * scl + group_sum<TPR>(ps);
            m_run = mn;
            _Float16 ph[CPS], pl[CPS];
#pragma unroll
            for (int e = 0; e < CPS; ++e) {
                ph[e] = (_Float16)p[e];
                pl[e] = (_Float16)(p[e] - (float)ph[e]);
            }
            __builtin_memcpy(&L.pt[0][sr][sc0], ph, sizeof(ph));
            __builtin_memcpy(&L.pt[1][sr][sc0], pl, sizeof(pl));
            if (t % TPR == 0)
                L.sc[sr] = scl;
        }
        // V into the tile (every read of K was before the barrier above);
        // rows of cells past the last are zeroed (weight 0 times anything)
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + kUT * r;
            *(u32x4 *)(L.ktile + (pr / CH) * VROW + 16 * ((pr % CH) ^ unit::vswz<DH>(pr / CH))) =
                kUC * it + pr / CH < ncells ? vc.template at<r>() : u32x4{0u, 0u, 0u, 0u};
        });
        load_rows(vp, it + 1, ia, vc);
        __syncthreads();                                                // barrier: weights, V tile
        // out^T = out^T * sc + V^T P: A = 16 dims x 32 cells down the V
        // tile's columns (one per 16-dim tile of the wave, shared by the row
        // tiles), B = 32 cells x 16 rows of a row tile, hi and lo
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float scl = 16 * rt + hn < R ? L.sc[16 * rt + hn] : 1.0f;
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[i][rt][q] *= scl;
        }
#pragma unroll
        for (int ks = 0; ks < kUC / 32; ++ks) {
            half8 a[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tile = wave + kUW * i;
                a[i] = half8{};
                if (NT % kUW == 0 || tile < NT) {
                    // a[i][e] = V[32 ks + 8 kq + e][16 tile + hn] by two transpose
                    // reads (rows 32 ks + 8 kq + e share one unit::vswz)
                    const int r0 = 32 * ks + 8 * kq + (hn >> 2);
                    const unsigned char *p0 = L.ktile + r0 * VROW +
                                              16 * ((2 * tile + ((hn & 3) >> 1)) ^ unit::vswz<DH>(r0)) + 8 * (hn & 1);
                    unit::lds_tr4(p0, a[i], 0);
                    unit::lds_tr4(p0 + 4 * VROW, a[i], 4);
                }
            }
            // (rows past the group's take whatever their weight rows hold:
            // only their own output columns see it, and those are not written)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                half8 bh, bl;
                __builtin_memcpy(&bh, &L.pt[0][16 * rt + hn][32 * ks + 8 * kq], 16);
                __builtin_memcpy(&bl, &L.pt[1][16 * rt + hn][32 * ks + 8 * kq], 16);
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int tile = wave + kUW * i;
                    if (NT % kUW == 0 || tile < NT) {
                        acc[i][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bh, acc[i][rt], 0, 0, 0);
                        acc[i][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bl, acc[i][rt], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();                                                // barrier: tile free
    };
    for (int32_t it = 0; it < nit; it += 2) {
        step(it, i1, i0);
        if (it + 1 < nit)
            step(it + 1, i0, i1);
    }

    // row r: query q0 + r / G, head g G + r % G
    if (sr < R && t % TPR == 0)
        L.lrow[sr] = l_run;
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 16 * rt + hn;
        if (r < R && r / G < nqg) {
            const int qi = r / G, h = r % G;
            const float l = L.lrow[r];
            float *o = c.out + ((size_t)(q0 + qi) * c.kv_heads * G + (size_t)g * G + h) * DH;
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tile = wave + kUW * i;
                if (NT % kUW != 0 && tile >= NT)
                    continue;
                const int d0 = 16 * tile + 4 * kq;
                *(float4 *)(o + d0) =
                    make_float4(acc[i][rt][0] / l, acc[i][rt][1] / l, acc[i][rt][2] / l, acc[i][rt][3] / l);
            }
        }
    }
}

template <int DH, int G, int RT>
hipError_t go(const ChunkArgs &c, int n_groups, hipStream_t s)
{
    const size_t lds = sizeof(ULds<DH, RT>);
    static_assert(sizeof(ULds<DH, RT>) <= 160 * 1024, "the LDS of one compute unit");
    static hipError_t attr = hipFuncSetAttribute((const void *)k_union_attend<DH, G, RT>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_union_attend<DH, G, RT>), dim3(n_groups, c.kv_heads), dim3(kUT), lds, s, c);
    return hipGetLastError();
}

template <int DH, int G>
hipError_t go_rt(const ChunkArgs &c, int n_groups, int RT, hipStream_t s)
{
    switch (RT) {
    case 1: return go<DH, G, 1>(c, n_groups, s);
    case 2: return go<DH, G, 2>(c, n_groups, s);
    case 4: return go<DH, G, 4>(c, n_groups, s);
    }
    return hipErrorInvalidValue;
}

template <int DH>
hipError_t go_g(const ChunkArgs &c, int n_groups, int G, int RT, hipStream_t s)
{
    switch (G) {
    case 1: return go_rt<DH, 1>(c, n_groups, RT, s);
    case 2: return go_rt<DH, 2>(c, n_groups, RT, s);
    case 4: return go_rt<DH, 4>(c, n_groups, RT, s);
    case 8: return go_rt<DH, 8>(c, n_groups, RT, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t union_build_lds(int qg, int32_t nb_last)
{
    return sizeof(uint32_t) * ((size_t)qg * ((nb_last + 31) / 32) + kUB / kWave);
}

hipError_t launch_union(const ChunkArgs &c, int Dh, int G, hipStream_t s)
{
    const int QG = c.union_q;
    if (QG < 1 || QG > kUnionMaxQ || QG * G > 16 * kMaxRT || c.ucap < QG * c.kb)
        return hipErrorInvalidValue;
    const int RT = QG * G <= 16 ? 1 : QG * G <= 32 ? 2 : 4;
    const int n_groups = (c.n_q + QG - 1) / QG;
    const size_t blds = union_build_lds(QG, c.nb_last);
    if (blds > kUnionBuildLds)
        return hipErrorInvalidValue;
    static hipError_t battr = hipFuncSetAttribute((const void *)k_union_build,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)kUnionBuildLds);
    if (battr != hipSuccess)
        return battr;
    hipLaunchKernelGGL(k_union_build, dim3(n_groups), dim3(kUB), blds, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (Dh) {
    case 64: return go_g<64>(c, n_groups, G, RT, s);
    case 128: return go_g<128>(c, n_groups, G, RT, s);
    case 256: return go_g<256>(c, n_groups, G, RT, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace qsa
