// qsa_unit.h -- the attention unit shared by the prefill chunk, the batched
// and multi-query decode, the masked ablation and the fused decode step: one
// query of one sequence, one KV head, a run of chosen cells in 64-cell
// iterations [post 10, "selected QSA K/V gather（COMMON-005）": only the K/V
// rows of the chosen cells are read, and ordinary softmax attention runs over
// them].
//
// Every thread loads K and V chunks of the iteration (coalesced: consecutive
// threads read consecutive bytes of a row) one iteration ahead; K goes to an
// LDS tile, where waves 0-3 take the 64 x G logits on the matrix cores (q as
// two f16 halves); waves h < G run the online softmax of head h over the 64
// cells and leave its weights in LDS as two f16 halves (hi + lo: V times
// either half is exact in fp32); V then takes the K tile's place, and P.V
// also runs on the matrix cores: out^T (dims x heads) += V^T (dims x cells)
// . P (cells x heads), wave w owning the 16-dim tiles w, w + NW, ... for the
// whole run, so no cross-wave sum is left at the end.
//
// Modes (which cells a unit takes):
//   kSplits  the query's chosen blocks (or every block) then its tail cells,
//            in 64-cell iterations dealt out to c.ns splits;
//   kMasked  every cell 0 .. n-1 is read; blocks whose bit in c.mask is
//            clear get logit -inf (the selection applied as a mask);
//   kOwn     the caller's block ids, already in L.ids[0 .. c.kb) (one split,
//            no tail); an id with its sign bit set is a block whose rows are
//            loaded but whose logits are -inf.  The caller also fills the
//            q operand (load_qb) before the unit's first barrier.
// COHERENT: the partial (m, l, acc) is written with device-coherent stores
// (read back inside the same kernel by another workgroup).
#pragma once
#include <type_traits>

#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {
namespace unit {

constexpr int kCI = kUnitCells;              // cells per iteration

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum Mode { kSplits = 0, kMasked = 1, kOwn = 2 };

// Up to eight registers named at compile time (arrays indexed in a loop that
// spans the iteration loop end up in scratch memory).
template <class T>
struct Regs8 {
    T x0, x1, x2, x3, x4, x5, x6, x7;
    template <int R>
    __device__ __forceinline__ T &at()
    {
        if constexpr (R == 0) return x0;
        else if constexpr (R == 1) return x1;
        else if constexpr (R == 2) return x2;
        else if constexpr (R == 3) return x3;
        else if constexpr (R == 4) return x4;
        else if constexpr (R == 5) return x5;
        else if constexpr (R == 6) return x6;
        else return x7;
    }
};

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// The LDS tile's 16-byte chunk c of row r sits at chunk c ^ swz(r): a P.V
// operand read takes one 2-byte column of rows 8 kq + e (kq < 4, e < 8), and
// with rows 2 DH + 16 bytes apart those four row groups would share banks;
// the swizzle puts them 32 bytes apart.  Every access to the tile (K and V
// writes, logit and P.V reads) goes through it.
__device__ __forceinline__ int swz(int r) { return 2 * ((r >> 3) & 3); }

// LDS transpose read of 16-bit values (gfx950): within each group of 16
// lanes, lane r names 4 consecutive values M[r][0..3] at p (8-byte aligned),
// and lane j receives M[4 i + j / 4][j % 4] for i = 0..3.
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 tr16x4;

__device__ __forceinline__ void lds_tr4(const unsigned char *p, half8 &a, int at)
{
    typedef __attribute__((address_space(3))) tr16x4 *lds_tr_ptr;
    const tr16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_tr_ptr)(p));
    _Float16 h[4];
    __builtin_memcpy(h, &v, 8);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        a[at + e] = h[e];
}

// The V tile's layout (head dims >= 128): rows 2 DH + 32 bytes apart, so that
// consecutive rows sit 32 bytes apart in the banks, and chunk c of row r at
// c ^ vswz(r), the two 8-chunk halves of a 16-chunk group swapped for rows
// with odd r / 8.  A P.V transpose read takes 32 bytes from each of 4
// consecutive rows per 16-lane group, and a half-wave's two groups take rows
// 8 apart: their 8 windows then fill the 64 banks once.  Head dim 64 (8
// chunks a row) keeps the K layout.
template <int DH>
__device__ __forceinline__ int vswz(int r)
{
    if constexpr (DH >= 128)
        return 8 * ((r >> 3) & 1);
    else
        return swz(r);
}

// K and V move in 16-byte chunks, both through the LDS tile.
template <int DH, int G, int NTH>
struct CAShape {
    static constexpr int NW = NTH / kWave;                // waves
    static constexpr int KCH = DH / 8;                    // 16-byte chunks of a K row
    static constexpr int KPAIRS = kCI * KCH;
    static constexpr int KR = (KPAIRS + NTH - 1) / NTH;   // K chunks per thread
    static constexpr int VCH = DH / 8;                    // 16-byte chunks of a V row
    static constexpr int VPAIRS = kCI * VCH;
    static constexpr int VR = (VPAIRS + NTH - 1) / NTH;   // V chunks per thread
    static constexpr int KS = DH / 32;                    // MFMA k-steps of a row
    static constexpr int KROW = 2 * DH + 16;              // padded LDS bytes of a K row
    static constexpr int VROW = DH >= 128 ? 2 * DH + 32 : KROW;   // and of a V row
    static constexpr int NT = DH / 16;                    // 16-dim output tiles of P.V
    static constexpr int TPW = (NT + NW - 1) / NW;        // tiles per wave
    static_assert(NTH % KCH == 0 && NTH % VCH == 0 && KPAIRS % kWave == 0 && VPAIRS % kWave == 0 &&
                  KR <= 8 && VR <= 8 && G <= NW && kCI / 16 <= NW, "shape");
};

template <int DH, int G>
struct CALds {
    static constexpr int KS = DH / 32;
    static constexpr int KROW = 2 * DH + 16;
    static constexpr int VROW = DH >= 128 ? 2 * DH + 32 : KROW;
    // the K tile, then (after the logits) the V tile of the iteration
    static constexpr int KT = kCI * (VROW > KROW ? VROW : KROW);
    alignas(16) unsigned char ktile[KT];
    alignas(16) uint4 qb[KS][2][kWave];
    float lg[kCI][G + 1];
    // softmax weights, hi and lo halves, [head][cell]: rows padded by 16
    // bytes, so that the heads of one P.V operand read fall 4 banks apart
    alignas(16) _Float16 pt[2][G][kCI + 8];
    float sc[G], mrow[G], lrow[G];
    int32_t ids[kChunkMaxIds];
};

// One attention unit: a query of one sequence, one KV head, one split.
struct QueryUnit {
    const uint16_t *k, *v;      // the sequence's K / V cache
    const int32_t *sel;         // its chosen block ids, ascending (null: every block kept)
    const float *q;             // [Hq][Dh]
    float *out;                 // [Hq][Dh], written when ns == 1
    float *part;                // [Hkv][ns] partials, written when ns > 1
    int64_t n;                  // tokens seen, the current one included
    int32_t kb;                 // blocks kept at most (kOwn: blocks in L.ids)
    int32_t kv_heads, ns;
    int32_t direct;             // ns == 1 and the output is written here, normalised
    float scale;
    const uint32_t *mask;       // kMasked: bit b set = block b takes part (every row is read)
};

// q of the G heads of KV head g as the B operand of the logit MFMA: lane l
// of k-step ks holds q[head l % 16][32 ks + 8 (l / 16) .. +8] (zero past G),
// hi and lo halves.  Whole workgroup (NTH threads) calls; no barrier.
template <int DH, int G, int NTH>
__device__ inline void load_qb(const float *q, CALds<DH, G> &L, int g)
{
    constexpr int KS = DH / 32;
    const float *qg = q + (size_t)g * G * DH;
    for (int x = threadIdx.x; x < KS * kWave; x += NTH) {
        const int ks = x / kWave, l = x % kWave, h = l % 16, d0 = 32 * ks + 8 * (l / 16);
        float4 u = make_float4(0.0f, 0.0f, 0.0f, 0.0f), v = u;
        if (h < G) {
            u = *(const float4 *)(qg + h * DH + d0);
            v = *(const float4 *)(qg + h * DH + d0 + 4);
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

template <bool COHERENT>
__device__ inline void put(float *p, float x)
{
    if constexpr (COHERENT)
        __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = x;
}

struct NoHook {
    __device__ void operator()() const {}
};

// Unit (split s, KV head g) of query c; see the modes above.  Whole
// workgroup (NTH threads) calls.  hook() runs once, by every thread, after
// the first iteration's K / V loads are issued and before any logit is
// taken (it may hold a barrier and may still change the sign bits of the
// kOwn ids: the rows are loaded either way).
template <int DH, int G, int NTH, int MODE, bool COHERENT = false, class Hook = NoHook>
__device__ void attend_unit(const QueryUnit &c, CALds<DH, G> &L, int s, int g, Hook hook = Hook())
{
    using S = CAShape<DH, G, NTH>;
    constexpr int KCH = S::KCH, VCH = S::VCH, KR = S::KR, VR = S::VR, KS = S::KS, KROW = S::KROW, VROW = S::VROW,
                  NT = S::NT, TPW = S::TPW, NW = S::NW;
    constexpr bool SIGNED = MODE != kSplits;        // ids carry a masked-out sign bit
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int ns = c.ns;
    const int64_t n = c.n;
    const int32_t nbq = (int32_t)(n >> 2);
    int32_t nsel, ncells, it0, it1, id0;
    if constexpr (MODE == kOwn) {
        nsel = c.kb;
        ncells = 4 * nsel;
        it0 = 0;
        it1 = (ncells + kCI - 1) / kCI;
        id0 = 0;
    } else {
        const bool keep_all = !c.sel || nbq <= c.kb;
        nsel = keep_all ? nbq : c.kb;
        ncells = 4 * nsel + (int32_t)(n & 3);
        const int32_t nit = (ncells + kCI - 1) / kCI;
        const int32_t ipw = (nit + ns - 1) / ns;
        it0 = s * ipw;
        it1 = it0 + ipw < nit ? it0 + ipw : nit;
        // the split's block ids (16 per iteration)
        id0 = (kCI / 4) * it0;
        const int32_t id1 = (kCI / 4) * it1 < nsel ? (kCI / 4) * it1 : nsel;
        const int32_t *srow = c.sel;
        for (int x = id0 + t; x < id1; x += NTH) {
            if constexpr (MODE == kMasked)   // the id, its sign bit set when the block is masked out
                L.ids[x - id0] = x | (((c.mask[x >> 5] >> (x & 31)) & 1u) ? 0 : (int32_t)0x80000000);
            else
                L.ids[x - id0] = keep_all ? x : srow[x];
        }
        load_qb<DH, G, NTH>(c.q, L, g);
    }
    __syncthreads();

    // Row of local cell lc of iteration it; invalid cells read row 0, masked.
    auto cell_row = [&](int it, int lc, bool &valid) __attribute__((always_inline)) -> size_t {
        const int32_t e = kCI * it + lc;
        valid = e < ncells;
        int64_t cell;
        if (e < 4 * nsel) {
            int32_t b = L.ids[(e >> 2) - id0];
            if constexpr (SIGNED) {     // a masked-out row is still loaded, its logit is -inf
                const bool live = valid;
                valid = valid && b >= 0;
                b &= 0x7FFFFFFF;
                cell = 4 * (int64_t)b + (e & 3);
                return live ? (size_t)cell : 0;
            }
            valid = valid && (uint32_t)b < (uint32_t)nbq;
            cell = 4 * (int64_t)b + (e & 3);
        } else {
            cell = 4 * (int64_t)nbq + (e - 4 * nsel);
        }
        return valid ? (size_t)cell : 0;
    };
    auto row_base = [&](int it, int lc) __attribute__((always_inline)) -> size_t {
        bool v;
        return (cell_row(it, lc, v) * c.kv_heads + g) * DH;
    };
    auto load_k = [&](int it, Regs8<u32x4> &kr) __attribute__((always_inline)) {
        static_for<KR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + NTH * r;
            if (pr < S::KPAIRS)
                kr.template at<r>() = *(const u32x4 *)(c.k + row_base(it, pr / KCH) + 8 * (pr % KCH));
        });
    };
    auto load_v = [&](int it, Regs8<u32x4> &vr) __attribute__((always_inline)) {
        static_for<VR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + NTH * r;
            if (pr < S::VPAIRS)
                vr.template at<r>() = *(const u32x4 *)(c.v + row_base(it, pr / VCH) + 8 * (pr % VCH));
        });
    };

    // P.V accumulators: wave w owns the 16-dim tiles w, w + NW, ...; lane l
    // holds out^T[dim 16 tile + 4 (l / 16) + j][head l % 16], j < 4
    const int hn = lane & 15, kq = lane >> 4;
    float4v acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
        acc[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;          // wave h < G: head h
    // K and V one iteration ahead: K leaves the registers for the LDS tile
    // first thing, V when the tile is free again (after the logits)
    Regs8<u32x4> kr;
    Regs8<u32x4> vr;
    if (it0 < it1) {
        load_k(it0, kr);
        load_v(it0, vr);
    }
    hook();

    for (int32_t it = it0; it < it1; ++it) {
        static_for<KR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + NTH * r;
            if (pr < S::KPAIRS)
                *(u32x4 *)(L.ktile + (pr / KCH) * KROW + 16 * ((pr % KCH) ^ swz(pr / KCH))) = kr.template at<r>();
        });
        if (it + 1 < it1)
            load_k(it + 1, kr);
        __syncthreads();
        if (wave < kCI / 16) {
            // D[cell][head] = K[cell][:] . q[head][:], 16 cells per wave
            const int mc = lane & 15, kg = lane >> 4;
            float4v d = {0.0f, 0.0f, 0.0f, 0.0f}, e = d;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                half8 a, bh, bl;
                __builtin_memcpy(&a, L.ktile + (16 * wave + mc) * KROW + 16 * ((4 * ks + kg) ^ swz(16 * wave + mc)), 16);
                __builtin_memcpy(&bh, &L.qb[ks][0][lane], 16);
                __builtin_memcpy(&bl, &L.qb[ks][1][lane], 16);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, d, 0, 0, 0);
                e = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, e, 0, 0, 0);
            }
            if (mc < G) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int lc = 16 * wave + 4 * kg + j;
                    bool v;
                    (void)cell_row(it, lc, v);
                    L.lg[lc][mc] = v ? c.scale * (d[j] + e[j]) : -INFINITY;
                }
            }
        }
        __syncthreads();
        if (wave < G) {
            // online softmax of head `wave` over the 64 cells (lane = cell)
            const float x = L.lg[lane][wave];
            const float mn = fmaxf(m_run, wave::reduce_max_f(x));
            float sc = 1.0f, pv = 0.0f;
            if (mn != -INFINITY) {
                sc = m_run == -INFINITY ? 0.0f : expf(m_run - mn);
                pv = x == -INFINITY ? 0.0f : expf(x - mn);
            }
            l_run = l_run * sc + wave::reduce_add_f(pv);
            m_run = mn;
            const _Float16 ph = (_Float16)pv;
            L.pt[0][wave][lane] = ph;
            L.pt[1][wave][lane] = (_Float16)(pv - (float)ph);
            if (lane == 0)
                L.sc[wave] = sc;
        }
        // V into the tile (every read of K was before the barrier above)
        static_for<VR>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int pr = t + NTH * r;
            if (pr < S::VPAIRS)
                *(u32x4 *)(L.ktile + (pr / VCH) * VROW + 16 * ((pr % VCH) ^ vswz<DH>(pr / VCH))) =
                    vr.template at<r>();
        });
        if (it + 1 < it1)
            load_v(it + 1, vr);
        __syncthreads();
        // out^T = out^T * sc + V^T P: A = 16 dims x 32 cells read down the V
        // tile's columns, B = 32 cells x 16 heads (zero past G), hi and lo
        const float scl = hn < G ? L.sc[hn] : 1.0f;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] *= scl;
#pragma unroll
        for (int ks = 0; ks < kCI / 32; ++ks) {
            half8 bh = {}, bl = {};
            if (hn < G) {
                __builtin_memcpy(&bh, &L.pt[0][hn][32 * ks + 8 * kq], 16);
                __builtin_memcpy(&bl, &L.pt[1][hn][32 * ks + 8 * kq], 16);
            }
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tile = wave + NW * i;
                if (NT % NW == 0 || tile < NT) {
                    // a[e] = V[32 ks + 8 kq + e][16 tile + hn]: two transpose
                    // reads, lane hn of the group naming row 8 kq + 4 h + hn / 4,
                    // dims 16 tile + 4 (hn % 4) .. +4 (rows 32 ks + 8 kq + e share
                    // one vswz)
                    half8 a;
                    const int r0 = 32 * ks + 8 * kq + (hn >> 2);
                    const unsigned char *p0 = L.ktile + r0 * VROW +
                                              16 * ((2 * tile + ((hn & 3) >> 1)) ^ vswz<DH>(r0)) + 8 * (hn & 1);
                    lds_tr4(p0, a, 0);
                    lds_tr4(p0 + 4 * VROW, a, 4);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, acc[i], 0, 0, 0);
                }
            }
        }
        __syncthreads();   // the tile takes the next iteration's K
    }

    if (wave < G && lane == 0) {
        L.mrow[wave] = m_run;
        L.lrow[wave] = l_run;
    }
    __syncthreads();
    float *part = c.part + ((size_t)g * ns + s) * (size_t)part_stride(G, DH);
    if (hn < G) {
        const float l = L.lrow[hn];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wave + NW * i;
            if (NT % NW != 0 && tile >= NT)
                continue;
            const int d0 = 16 * tile + 4 * kq;
            if (c.direct) {
                float *o = c.out + ((size_t)g * G + hn) * DH + d0;
                *(float4 *)o = make_float4(acc[i][0] / l, acc[i][1] / l, acc[i][2] / l, acc[i][3] / l);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)            // a partial's stride is not a multiple of 4
                    put<COHERENT>(part + 2 * G + hn * DH + d0 + j, acc[i][j]);
            }
        }
    }
    if (!c.direct && wave == 0 && lane < G) {
        put<COHERENT>(part + lane, L.mrow[lane]);
        put<COHERENT>(part + G + lane, L.lrow[lane]);
    }
}

}  // namespace unit
}  // namespace qsa
