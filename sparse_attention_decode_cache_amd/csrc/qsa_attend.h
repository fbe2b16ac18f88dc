// qsa_attend.h -- device code of stage 4 shared by the decode and chunk
// attention kernels: the attention of one 16-cell tile of one KV head for all
// G query heads of its group.
//
// [post 10, "selected QSA K/V gather（COMMON-005）"]: only the K/V rows of the
// chosen cells (4 per chosen block, plus the tail of the unfinished block) are
// read, and ordinary softmax attention runs over them.  1024 threads; every K
// and V load of a tile is issued at once:
//   wave 0 (QK): the 16 x G logits on the matrix cores, K rows fed straight
//              from memory as the A operand, q (split into two f16 halves)
//              as B;
//   softmax:   one 16-lane DPP row per head (16 cells);
//   waves 8-15 (PV): a lane owns (8-dim chunk, head, cell group) and keeps
//              the V chunks of its cells in registers (coalesced: a wave-wide
//              load covers whole rows); partial sums of the cell groups meet
//              in LDS and are summed in a fixed order.
#pragma once
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {
namespace att {


typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kAT = 1024;                   // threads of an attention workgroup
constexpr int kCells = kCellsPerSplit;      // cells per workgroup (16: one MFMA tile)
constexpr int kPV0 = kAT / 2;               // PV lanes [512, 1024)
static_assert(kCells == 16, "one 16x16 MFMA tile of cells, one 16-lane row per softmax");

typedef float float4v __attribute__((ext_vector_type(4)));

template <int DH, int G>
struct AttShape {
    static constexpr int KS = DH / 32;                      // MFMA k-steps of a row
    static constexpr int CH = DH / 8;                       // 16-byte chunks of a row
    static constexpr int SV0 = (kAT - kPV0) / (CH * G);
    static constexpr int SV = SV0 < kCells ? SV0 : kCells;  // cell groups of the PV lanes
    static constexpr int PV_LANES = SV * CH * G;
    static constexpr int CPG = kCells / SV;                 // cells per PV lane
    static_assert(G <= 16 && CPG * SV == kCells && PV_LANES <= kAT - kPV0, "shape");
};

template <int DH, int G>
struct AttLds {
    using S = AttShape<DH, G>;
    float lg[kCells][G + 1];
    float m[G], l[G];
    alignas(16) float acc[S::SV][G * DH];
    int32_t blk[kCells / 4];
};

// Scales of a q8_0 K/V cache ([rows][kv_heads][DH/32] binary16); a.k and a.v
// then point at the int8 codes ([rows][kv_heads][DH]).
struct Q8Scales {
    const uint16_t *k = nullptr, *v = nullptr;
};

// Attention of the 16 cells e0 .. e0+15 of KV head g; blk[0..4) holds their
// 4 block ids (read only for cells inside the chosen blocks) and is visible to
// all threads.  The tile's (m[G], l[G], acc[G][DH]) end in L.m, L.l and the
// L.acc groups; sink(L) consumes them after the last barrier (every thread
// calls it).  Whole workgroup calls.
//
// Q8: K and V are q8_0 rows (code * scale, one scale per 32 values).  An MFMA
// k-step spans 32 dims, one q8_0 block: the codes (exact in f16) meet q on
// the matrix cores and each k-step's partial logit is multiplied by its
// cell's scale in fp32; the PV lanes decode their 8 values in fp32.
template <int DH, int G, bool Q8 = false, class Sink>
__device__ void attend_tile(const AttendArgs &a, AttLds<DH, G> &L, const int32_t *blk, int e0, int g,
                            Sink sink, Q8Scales q8 = {})
{
    using S = AttShape<DH, G>;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;

    // Row of local cell lc; invalid cells (past n_cells, or a block id
    // outside [0, nb)) read row 0 and are masked.
    auto cell_row = [&](int lc, bool &valid) -> size_t {
        const int e = e0 + lc;
        valid = e < a.n_cells;
        int64_t cell;
        if (e < 4 * a.n_sel_blocks) {
            const int32_t b = blk[lc >> 2];
            valid = valid && (uint32_t)b < (uint32_t)a.nb;
            cell = 4 * (int64_t)b + (lc & 3);
        } else {
            cell = 4 * (int64_t)a.nb + (e - 4 * a.n_sel_blocks);
        }
        return valid ? (size_t)cell : 0;
    };

    const int tv = t - kPV0;
    const int v_chunk = tv % S::CH, v_head = (tv / S::CH) % G, v_grp = tv / (S::CH * G);
    uint4 vr[S::CPG];
    [[maybe_unused]] float vs[S::CPG];      // Q8: the V scales of the lane's cells

    if (wave == 0) {
        // ---- logits on the matrix cores: D[cell][head] = K[cell][:] . q[head][:]
        // 16x16x32 f16 MFMA: lane l feeds A[cell l%16][8(l/16) .. +8] (K row)
        // and B[8(l/16) .. +8][head l%16] (q, zero past G), and receives
        // D[4(l/16) + j][l%16].  q = hi + lo in f16, both multiplied: the
        // products are exact in fp32, so the dot keeps fp32 accuracy.
        const int mc = lane & 15, kg = lane >> 4;
        bool valid;
        const size_t row = cell_row(mc, valid);
        uint4 kr[S::KS];
        [[maybe_unused]] float ks[S::KS];   // Q8: row mc's scale of k-step i
        if constexpr (Q8) {
            const int8_t *kp = (const int8_t *)a.k + (row * a.kv_heads + g) * DH + 8 * kg;
            const uint16_t *sp = q8.k + (row * a.kv_heads + g) * (DH / 32);
#pragma unroll
            for (int i = 0; i < S::KS; ++i) {
                const uint2 w = *(const uint2 *)(kp + 32 * i);
                kr[i] = make_uint4(w.x, w.y, 0u, 0u);
                ks[i] = (float)__builtin_bit_cast(_Float16, sp[i]);
            }
        } else {
            const uint4 *kp = (const uint4 *)(a.k + (row * a.kv_heads + g) * DH) + kg;
#pragma unroll
            for (int i = 0; i < S::KS; ++i)
                kr[i] = kp[4 * i];
        }
        const bool hq = mc < G;
        const float4 *qp = (const float4 *)(a.q + ((size_t)g * G + (hq ? mc : 0)) * DH) + 2 * kg;
        float4 qx[S::KS], qy[S::KS];
#pragma unroll
        for (int i = 0; i < S::KS; ++i) {
            qx[i] = qp[8 * i];
            qy[i] = qp[8 * i + 1];
        }
        // every K / q load above is in flight before the first use: left to
        // itself the scheduler sinks some of them into the MFMA chain, which
        // then waits out one memory round trip after another
        __builtin_amdgcn_sched_barrier(0);
        float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < S::KS; ++i) {
            const float4 x = qx[i], y = qy[i];
            const float qf[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            half8 hi, lo, kh;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q = hq ? qf[j] : 0.0f;
                hi[j] = (_Float16)q;
                lo[j] = (_Float16)(q - (float)hi[j]);
            }
            if constexpr (Q8) {
                // D[4kg + j][mc] += scale(cell 4kg + j, k-step i) * (codes . q)
                int8_t c8[8];
                __builtin_memcpy(c8, &kr[i], 8);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    kh[j] = (_Float16)c8[j];
                float4v p = {0.0f, 0.0f, 0.0f, 0.0f};
                p = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, hi, p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, lo, p, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    d[j] = fmaf(__shfl(ks[i], 4 * kg + j), p[j], d[j]);
            } else {
                __builtin_memcpy(&kh, &kr[i], 16);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, hi, d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, lo, d, 0, 0, 0);
            }
        }
        if (hq) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int lc = 4 * kg + j;
                bool v;
                (void)cell_row(lc, v);
                L.lg[lc][mc] = v ? a.scale * d[j] : -INFINITY;
            }
        }
    } else if (tv >= 0 && tv < S::PV_LANES) {
#pragma unroll
        for (int i = 0; i < S::CPG; ++i) {
            bool valid;
            const size_t row = cell_row(v_grp + S::SV * i, valid);
            if constexpr (Q8) {
                const size_t rb = row * a.kv_heads + g;
                const uint2 w = *(const uint2 *)((const int8_t *)a.v + rb * DH + v_chunk * 8);
                vr[i] = make_uint4(w.x, w.y, 0u, 0u);
                vs[i] = (float)__builtin_bit_cast(_Float16, q8.v[rb * (DH / 32) + v_chunk / 4]);
            } else {
                vr[i] = *(const uint4 *)(a.v + (row * a.kv_heads + g) * DH + v_chunk * 8);
            }
        }
    }
    __syncthreads();

    // ---- softmax over the 16 cells, head = wave, cells = lanes 0-15 (row 0)
    if (wave < G) {
        const float x = L.lg[lane & 15][wave];
        const float m = wave::row_max_f(x);          // -inf only if no cell is valid
        const float p = x == -INFINITY ? 0.0f : expf(x - m);
        const float l = wave::row_sum_f(p);
        if (lane < kCells)
            L.lg[lane][wave] = p;
        if (lane == 0) {
            L.m[wave] = m;
            L.l[wave] = l;
        }
    }
    __syncthreads();

    // ---- P . V over this lane's cells
    if (tv >= 0 && tv < S::PV_LANES) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < S::CPG; ++i) {
            const float p = L.lg[v_grp + S::SV * i][v_head];
            if constexpr (Q8) {
                int8_t c8[8];
                __builtin_memcpy(c8, &vr[i], 8);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = fmaf(p, (float)c8[j] * vs[i], acc[j]);
            } else {
                half8 vh;
                __builtin_memcpy(&vh, &vr[i], 16);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = fmaf(p, (float)vh[j], acc[j]);
            }
        }
        float4 *dst = (float4 *)&L.acc[v_grp][v_head * DH + v_chunk * 8];
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    sink(L);
}

// Sum of the PV cell groups for element i = h*DH + d (fixed order).
template <int DH, int G>
__device__ inline float tile_acc(const AttLds<DH, G> &L, int i)
{
    float s = L.acc[0][i];
#pragma unroll
    for (int grp = 1; grp < AttShape<DH, G>::SV; ++grp)
        s += L.acc[grp][i];
    return s;
}

}  // namespace att
}  // namespace qsa
