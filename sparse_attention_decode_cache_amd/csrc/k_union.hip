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
// A group is as many queries as fill the 16 rows of one matrix-core tile:
// QG = 16 / G queries of G heads each (fewer when QG K ids would not fit).
//   build   one workgroup per group: the queries' ids as bitmaps in LDS, OR-ed
//           and compacted in ascending order into the group's union list,
//           with each union block's mask of the queries that chose it;
//   attend  workgroup (group, KV head), 512 threads: the union's cells (4 per
//           block, ascending) and then the group's tail range [4 floor(n_first
//           / 4), n_last), 64 cells per iteration: K and V rows land in an LDS
//           tile once for the whole group; the logits of all QG x G rows on
//           the matrix cores (q as f16 hi + lo), a cell counting for a row
//           only if it is that query's own; online softmax per row; P.V on
//           the matrix cores; the output written normalised per query.
#include "qsa_internal.h"
#include "qsa_unit.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

constexpr int kUB = 512;                     // build threads
constexpr int kUT = 512;                     // attend threads
constexpr int kUW = kUT / kWave;
constexpr int kUC = 64;                      // cells per iteration
constexpr int kRows = 16;                    // query x head rows of a group

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

template <int DH>
struct UShape {
    static constexpr int KS = DH / 32;              // MFMA k-steps of a row
    static constexpr int KROW = 2 * DH + 16;        // padded LDS bytes of a K / V row
    static constexpr int CH = DH / 8;               // 16-byte chunks of a row
    static constexpr int PAIRS = kUC * CH;          // (cell, chunk) pairs of an iteration
    static constexpr int PR = PAIRS / kUT;
    static_assert(PAIRS % kUT == 0 && PR <= 8, "whole (cell, chunk) pairs per thread, at most 8");
    static constexpr int NT = DH / 16;              // 16-dim output tiles
    static constexpr int TPW = (NT + kUW - 1) / kUW;
};

template <int DH>
struct ULds {
    using S = UShape<DH>;
    alignas(16) unsigned char ktile[kUC * S::KROW];   // K, then V, of the iteration
    alignas(16) uint4 qb[S::KS][2][kWave];
    float lg[kUC][kRows + 1];
    alignas(16) _Float16 pt[2][kRows][kUC];
    float sc[kRows], lrow[kRows];
    int32_t ids[kChunkMaxIds];
    uint32_t msk[kChunkMaxIds];
};

template <int DH, int G>
__global__ __launch_bounds__(kUT) void k_union_attend(ChunkArgs c)
{
    using S = UShape<DH>;
    constexpr int KS = S::KS, KROW = S::KROW, CH = S::CH, PR = S::PR, NT = S::NT, TPW = S::TPW;
    extern __shared__ uint4 ua_lds[];
    ULds<DH> &L = *reinterpret_cast<ULds<DH> *>(ua_lds);
    const int QG = c.union_q;
    const int R = QG * G;                          // rows in use (<= 16)
    const int j = blockIdx.x, g = blockIdx.y, q0 = j * QG;
    const int nqg = c.n_q - q0 < QG ? c.n_q - q0 : QG;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int32_t nu = c.ucount[j];
    const int64_t n_first = (int64_t)c.n0 + q0 + 1, n_last = (int64_t)c.n0 + q0 + nqg;
    const int64_t t0 = n_first / 4 * 4;
    const int32_t ncells = 4 * nu + (int32_t)(n_last - t0);
    const int32_t nit = (ncells + kUC - 1) / kUC;
    for (int x = t; x < nu; x += kUT) {
        L.ids[x] = c.uni[(size_t)j * c.ucap + x];
        L.msk[x] = c.umask[(size_t)j * c.ucap + x];
    }
    // q of the group's rows (query r / G, head g G + r % G) as the logit
    // MFMA's B operand: lane l of k-step ks holds row l % 16, dims 32 ks + 8
    // (l / 16) .. +8, zero past the rows in use
    for (int x = t; x < KS * kWave; x += kUT) {
        const int ks = x / kWave, l = x % kWave, r = l % 16, d0 = 32 * ks + 8 * (l / 16);
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
        __builtin_memcpy(&L.qb[ks][0][l], &hi, 16);
        __builtin_memcpy(&L.qb[ks][1][l], &lo, 16);
    }
    __syncthreads();

    // whether union position e is one of row r's query's own cells
    const uint32_t *msk = L.msk;
    auto own = [=](int32_t e, int r) -> bool {
        const int qi = r / G;
        if (e >= ncells || r >= R || qi >= nqg)
            return false;
        if (e < 4 * nu)
            return ((msk[e >> 2] >> qi) & 1u) != 0u;
        const int64_t cell = t0 + (e - 4 * nu), ni = n_first + qi;
        return cell >= ni / 4 * 4 && cell < ni;
    };
    const int hn = lane & 15, kq = lane >> 4;
    float4v acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
        acc[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    // wave w runs the softmax of rows w and w + 8
    float m_run0 = -INFINITY, m_run1 = -INFINITY, l_run0 = 0.0f, l_run1 = 0.0f;
    // K and V one iteration ahead, in registers named at compile time (an
    // array indexed across the iteration loop ends up in scratch memory):
    // thread t takes the (cell, chunk) pairs t + 512 r
    // (the lambdas see copies of the kernel arguments they use: taking the
    // address of the argument block would copy it to scratch memory)
    const uint16_t *kp = c.k, *vp = c.v;
    const int kvh = c.kv_heads;
    const int32_t *ids = L.ids;
    auto row_base = [=](int it, int pr) __attribute__((always_inline)) -> size_t {
        const int32_t e = kUC * it + pr / CH;
        int64_t cell = 0;
        if (e < ncells)
            cell = e < 4 * nu ? 4 * (int64_t)ids[e >> 2] + (e & 3) : t0 + (e - 4 * nu);
        return ((size_t)cell * kvh + g) * DH + 8 * (pr % CH);
    };
    auto load_k = [=](int it, unit::Regs8<u32x4> &kr) __attribute__((always_inline)) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            kr.template at<r>() = *(const u32x4 *)(kp + row_base(it, t + kUT * r));
        });
    };
    auto load_v = [=](int it, unit::Regs8<u32x4> &vr) __attribute__((always_inline)) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            vr.template at<r>() = *(const u32x4 *)(vp + row_base(it, t + kUT * r));
        });
    };
    unit::Regs8<u32x4> kr, vr;
    if (nit > 0) {
        load_k(0, kr);
        load_v(0, vr);
    }
    for (int32_t it = 0; it < nit; ++it) {
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + kUT * r;
            *(u32x4 *)(L.ktile + (pr / CH) * KROW + 16 * (pr % CH)) = kr.template at<r>();
        });
        if (it + 1 < nit)
            load_k(it + 1, kr);
        __syncthreads();                                                // barrier: K tile
        if (wave < kUC / 16) {
            // D[cell][row] = K[cell][:] . q[row][:], 16 cells per wave
            const int mc = lane & 15, kg = lane >> 4;
            float4v d = {0.0f, 0.0f, 0.0f, 0.0f}, ee = d;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                half8 a, bh, bl;
                __builtin_memcpy(&a, L.ktile + (16 * wave + mc) * KROW + 2 * (32 * ks + 8 * kg), 16);
                __builtin_memcpy(&bh, &L.qb[ks][0][lane], 16);
                __builtin_memcpy(&bl, &L.qb[ks][1][lane], 16);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, d, 0, 0, 0);
                ee = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, ee, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lc = 16 * wave + 4 * kg + q;
                L.lg[lc][mc] = own(kUC * it + lc, mc) ? c.scale * (d[q] + ee[q]) : -INFINITY;
            }
        }
        __syncthreads();                                                // barrier: logits
        // online softmax of rows wave and wave + 8 over the 64 cells (lane = cell)
#define QSA_UNION_SOFTMAX_ROW(r, m_run, l_run)                                          \
    do {                                                                                \
        const float x_ = L.lg[lane][r];                                                 \
        const float mn_ = fmaxf(m_run, wave::reduce_max_f(x_));                         \
        float scl_ = 1.0f, pv_ = 0.0f;                                                  \
        if (mn_ != -INFINITY) {                                                         \
            scl_ = m_run == -INFINITY ? 0.0f : expf(m_run - mn_);                       \
            pv_ = x_ == -INFINITY ? 0.0f : expf(x_ - mn_);                              \
        }                                                                               \
        l_run = l_run * scl_ + wave::reduce_add_f(pv_);                                 \
        m_run = mn_;                                                                    \
        const _Float16 ph_ = (_Float16)pv_;                                             \
        L.pt[0][r][lane] = ph_;                                                         \
        L.pt[1][r][lane] = (_Float16)(pv_ - (float)ph_);                                \
        if (lane == 0)                                                                  \
            L.sc[r] = scl_;                                                             \
    } while (0)
        if (wave < R)
            QSA_UNION_SOFTMAX_ROW(wave, m_run0, l_run0);
        if (wave + kUW < R)
            QSA_UNION_SOFTMAX_ROW(wave + kUW, m_run1, l_run1);
#undef QSA_UNION_SOFTMAX_ROW
        // V into the tile (every read of K was before the barrier above);
        // rows of cells past the last are zeroed (weight 0 times anything)
        unit::static_for<PR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + kUT * r;
            *(u32x4 *)(L.ktile + (pr / CH) * KROW + 16 * (pr % CH)) =
                kUC * it + pr / CH < ncells ? vr.template at<r>() : u32x4{0u, 0u, 0u, 0u};
        });
        if (it + 1 < nit)
            load_v(it + 1, vr);
        __syncthreads();                                                // barrier: weights, V tile
        // out^T = out^T * sc + V^T P: A = 16 dims x 32 cells down the V
        // tile's columns, B = 32 cells x 16 rows, hi and lo
        const float scl = hn < R ? L.sc[hn] : 1.0f;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[i][q] *= scl;
#pragma unroll
        for (int ks = 0; ks < kUC / 32; ++ks) {
            half8 bh = {}, bl = {};
            if (hn < R) {
                __builtin_memcpy(&bh, &L.pt[0][hn][32 * ks + 8 * kq], 16);
                __builtin_memcpy(&bl, &L.pt[1][hn][32 * ks + 8 * kq], 16);
            }
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tile = wave + kUW * i;
                if (NT % kUW == 0 || tile < NT) {
                    half8 a;
                    const unsigned char *col = L.ktile + (32 * ks + 8 * kq) * KROW + 2 * (16 * tile + hn);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        a[e] = *(const _Float16 *)(col + e * KROW);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, acc[i], 0, 0, 0);
                }
            }
        }
        __syncthreads();                                                // barrier: tile free
    }

    // row r: query q0 + r / G, head g G + r % G
    if (lane == 0 && wave < R)
        L.lrow[wave] = l_run0;
    if (lane == 0 && wave + kUW < R)
        L.lrow[wave + kUW] = l_run1;
    __syncthreads();
    if (hn < R && hn / G < nqg) {
        const int qi = hn / G, h = hn % G;
        const float l = L.lrow[hn];
        float *o = c.out + ((size_t)(q0 + qi) * c.kv_heads * G + (size_t)g * G + h) * DH;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wave + kUW * i;
            if (NT % kUW != 0 && tile >= NT)
                continue;
            const int d0 = 16 * tile + 4 * kq;
            *(float4 *)(o + d0) = make_float4(acc[i][0] / l, acc[i][1] / l, acc[i][2] / l, acc[i][3] / l);
        }
    }
}

template <int DH, int G>
hipError_t go(const ChunkArgs &c, int n_groups, hipStream_t s)
{
    const size_t lds = sizeof(ULds<DH>);
    static hipError_t attr = hipFuncSetAttribute((const void *)k_union_attend<DH, G>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_union_attend<DH, G>), dim3(n_groups, c.kv_heads), dim3(kUT), lds, s, c);
    return hipGetLastError();
}

template <int DH>
hipError_t go_g(const ChunkArgs &c, int n_groups, int G, hipStream_t s)
{
    switch (G) {
    case 1: return go<DH, 1>(c, n_groups, s);
    case 2: return go<DH, 2>(c, n_groups, s);
    case 4: return go<DH, 4>(c, n_groups, s);
    case 8: return go<DH, 8>(c, n_groups, s);
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
    if (QG < 1 || QG * G > kRows || (int64_t)QG * c.kb > kChunkMaxIds || c.ucap < QG * c.kb)
        return hipErrorInvalidValue;
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
    case 64: return go_g<64>(c, n_groups, G, s);
    case 128: return go_g<128>(c, n_groups, G, s);
    case 256: return go_g<256>(c, n_groups, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace qsa
