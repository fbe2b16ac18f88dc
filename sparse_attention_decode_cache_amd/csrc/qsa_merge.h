// qsa_merge.h -- the merge of split-attention partials, shared by the decode,
// batched, multi-query and chunk paths [post 10, "selected QSA K/V
// gather（COMMON-005）": softmax attention over the gathered cells, here
// computed in splits and combined exactly].
#pragma once
#include "qsa_attend.h"
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {
namespace mrg {

// A partial element: a plain load, or a device-coherent one when the
// partial was written inside the same kernel by another workgroup.
template <bool COHERENT>
__device__ inline float get(const float *p)
{
    if constexpr (COHERENT)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

// out[h][d] = sum_s e^(m_s - M) acc_s[h][d] / sum_s e^(m_s - M) l_s.
// Workgroup (h, 64-dim slice), 16 waves, one global latency round: thread s
// loads m_s while wave w loads (l_s, acc_s[d]) of splits w, w+16, ...; M by
// a block max; thread s turns m_s into the weight e^(m_s - M) in LDS; each
// wave sums its splits, and wave 0 sums the 16 wave results in order and
// adds the tail: a fixed order, bitwise repeatable.  The tail (cells
// 4*nb + j, j < n_tail, when the splits hold only the chosen blocks) is one
// more partial that wave 0 computes itself: <= 3 logits, its K/V rows
// loaded with the first round.
constexpr int kMT = 1024;
constexpr int kMW = kMT / kWave;
constexpr int kMRound = 8;                  // splits per wave per load round
constexpr int kMaxSplits = kMT;

struct MergeLds {
    float w[kMaxSplits];
    float red[kMW];
    float l[kMW], acc[kMW][kWave];
};

// Output unit (query head h, 64-dim slice ds) from the split partials and the
// tail.  Whole workgroup (kMT threads) calls.  Q8: the tail rows are q8_0
// (codes in a.k / a.v, scales in q8), read as code * scale.
template <int DH, int G, bool Q8 = false, bool COHERENT = false>
__device__ void merge_unit(const AttendArgs &a, MergeLds &ml, int h, int ds, att::Q8Scales q8 = {})
{
    float *s_w = ml.w, *s_red = ml.red, *s_l = ml.l;
    auto &s_acc = ml.acc;
    constexpr int QD = DH / kWave;              // dims per lane of a tail logit
    const int g = h / G, hh = h % G;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int ns = a.n_split;
    const size_t ps = (size_t)part_stride(G, DH);
    const float *base = a.part + (size_t)g * ns * ps;
    const int d = ds * kWave + lane;

    // m_s first, without a branch (threads past the splits read split 0 and
    // drop it), then the first round of (l, acc) loads: every load in flight
    // before anything waits
    float ms = get<COHERENT>(base + (size_t)(t < ns ? t : 0) * ps + hh);
    float l[kMRound], x[kMRound];
#pragma unroll
    for (int i = 0; i < kMRound; ++i) {
        const int s = wave + i * kMW;
        const float *p = base + (size_t)(s < ns ? s : 0) * ps;
        l[i] = get<COHERENT>(p + G + hh);
        x[i] = get<COHERENT>(p + 2 * G + hh * DH + d);
    }
    // the tail's K and V rows (wave 0): every load issued at once, rows past
    // the tail clamped to row 0 and masked below
    const int nt = wave == 0 ? a.n_tail : 0;
    float kq[3][QD], vt[3], qv[QD];
    if (nt) {
        // raw elements (f16, or q8_0 code and scale) loaded first, converted
        // after the barrier: a conversion scheduled between the loads would
        // wait for every load before it
        uint16_t kh[3][QD], vh[3], ksc[3][QD], vsc[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const size_t cell = j < nt ? 4 * (size_t)a.nb + j : 0;   // row 0: always there
            const size_t rb = cell * a.kv_heads + g;
            if constexpr (Q8) {
                const int8_t *kr = (const int8_t *)a.k + rb * DH;
                const int8_t *vr = (const int8_t *)a.v + rb * DH;
                const uint16_t *ks = q8.k + rb * (DH / 32), *vs = q8.v + rb * (DH / 32);
#pragma unroll
                for (int i = 0; i < QD; ++i) {
                    kh[j][i] = (uint16_t)(uint8_t)kr[lane + kWave * i];
                    ksc[j][i] = ks[(lane + kWave * i) / 32];
                }
                vh[j] = (uint16_t)(uint8_t)vr[d];
                vsc[j] = vs[d / 32];
            } else {
                const uint16_t *kr = a.k + rb * DH;
                const uint16_t *vr = a.v + rb * DH;
#pragma unroll
                for (int i = 0; i < QD; ++i)
                    kh[j][i] = kr[lane + kWave * i];
                vh[j] = vr[d];
            }
        }
#pragma unroll
        for (int i = 0; i < QD; ++i)
            qv[i] = a.q[(size_t)h * DH + lane + kWave * i];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if constexpr (Q8) {
#pragma unroll
                for (int i = 0; i < QD; ++i)
                    kq[j][i] = (float)(int8_t)(uint8_t)kh[j][i] *
                               (float)__builtin_bit_cast(_Float16, ksc[j][i]);
                vt[j] = (float)(int8_t)(uint8_t)vh[j] * (float)__builtin_bit_cast(_Float16, vsc[j]);
            } else {
#pragma unroll
                for (int i = 0; i < QD; ++i)
                    kq[j][i] = (float)__builtin_bit_cast(_Float16, kh[j][i]);
                vt[j] = (float)__builtin_bit_cast(_Float16, vh[j]);
            }
        }
    }

    if (t >= ns)
        ms = -INFINITY;
    float wm = wave::reduce_max_f(ms);
    float mt = -INFINITY, lt = 0.0f, at = 0.0f;
    if (nt) {
        // wave-uniform: the tail's logits, max, sum and this lane's dim
        float xl[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            float dp = 0.0f;
#pragma unroll
            for (int i = 0; i < QD; ++i)
                dp = fmaf(qv[i], kq[j][i], dp);
            xl[j] = a.scale * wave::reduce_add_f(dp);
            if (j < nt)
                mt = fmaxf(mt, xl[j]);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < nt) {
                const float pj = expf(xl[j] - mt);
                lt += pj;
                at = fmaf(pj, vt[j], at);
            }
        wm = fmaxf(wm, mt);
    }
    if (lane == 0)
        s_red[wave] = wm;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < kMW; ++w)
        M = fmaxf(M, s_red[w]);
    if (t < ns)
        s_w[t] = ms == -INFINITY ? 0.0f : expf(ms - M);
    __syncthreads();

    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kMRound; ++i) {
        const int s = wave + i * kMW;
        if (s < ns) {
            acc = fmaf(s_w[s], x[i], acc);
            lsum = fmaf(s_w[s], l[i], lsum);
        }
    }
    for (int s0 = wave + kMRound * kMW; s0 < ns; s0 += kMRound * kMW) {
#pragma unroll
        for (int i = 0; i < kMRound; ++i) {
            const int s = s0 + i * kMW;
            const float *p = base + (size_t)(s < ns ? s : 0) * ps;
            l[i] = get<COHERENT>(p + G + hh);
            x[i] = get<COHERENT>(p + 2 * G + hh * DH + d);
        }
#pragma unroll
        for (int i = 0; i < kMRound; ++i) {
            const int s = s0 + i * kMW;
            if (s < ns) {
                acc = fmaf(s_w[s], x[i], acc);
                lsum = fmaf(s_w[s], l[i], lsum);
            }
        }
    }
    if (lane == 0)
        s_l[wave] = lsum;
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        float A = s_acc[0][lane], L = s_l[0];
#pragma unroll
        for (int w = 1; w < kMW; ++w) {
            A += s_acc[w][lane];
            L += s_l[w];
        }
        if (nt) {
            const float wt = expf(mt - M);
            A = fmaf(wt, at, A);
            L = fmaf(wt, lt, L);
        }
        a.out[(size_t)h * DH + d] = A / L;
    }
}

}  // namespace mrg
}  // namespace qsa
