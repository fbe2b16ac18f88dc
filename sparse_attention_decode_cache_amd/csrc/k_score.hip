// k_score.hip -- stage 2: stream every cached summary row once and score it.
//
// s[b] = sum_h w[h] * <q_idx[h], summary[b][h]>   [post 10, "QSA indexer"]
//
// This is the only pass whose bytes grow with context (N_b rows of up to 1 KB),
// so it is written as a pure HBM stream: each lane owns one 16-byte chunk of a
// row (LPR lanes cover a row, 64/LPR rows per wave-wide load), a wave issues
// all T loads of its tile before using any (non-temporal: the rows are not
// reused in this step), and the per-row partial dot products are reduced with
// a transposing butterfly -- log2(LPR) exchange rounds for T rows instead of
// log2(LPR) rounds per row.  w[h] is folded into q_idx once per lane.
// Optional outputs: fp32 scores, order-preserving 32-bit keys and a histogram
// of the keys' top 12 bits (the first radix digit of the top-k).
#include "qsa_internal.h"

namespace qsa {
namespace {

// Transposing butterfly over the lanes of one row group.  Before: v[0..CNT)
// are partial sums of CNT different rows.  After: v[0] holds the full sum of
// row index `toff` (lanes that end with equal `toff` hold equal sums).
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
                v[k] = keep + __shfl_xor(send, O);
            }
            if (up)
                toff += H;
            Butterfly<O / 2, H>::run(v, lane, toff);
        } else {
            v[0] += __shfl_xor(v[0], O);
            Butterfly<O / 2, 1>::run(v, lane, toff);
        }
    }
};

__device__ inline uint32_t score_key(float s)
{
    // -0 and +0 must compare equal: canonicalise before taking the bits.
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool F16, int LPR>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a)
{
    constexpr int EPL = F16 ? 8 : 4;           // elements per 16-byte chunk
    constexpr int RPL = kWave / LPR;           // rows per wave-wide load
    constexpr int T = LPR < 16 ? LPR : 16;     // loads in flight per lane
    constexpr int RPW = T * RPL;               // rows per wave tile
    constexpr int ROWB = LPR * 16;             // row bytes

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = lane % LPR;
    const int sub = lane / LPR;
    const int64_t base = ((int64_t)blockIdx.x * 4 + wave) * RPW;
    if (base >= a.nb)
        return;

    float qw[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const int e = chunk * EPL + k;
        qw[k] = a.q[e] * a.w[e / a.D];
    }

    const char *rows = (const char *)a.summary;
    u32x4 buf[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int64_t r = base + (int64_t)t * RPL + sub;
        if (r < a.nb)
            buf[t] = __builtin_nontemporal_load((const u32x4 *)(rows + r * ROWB) + chunk);
        else
            buf[t] = u32x4{0u, 0u, 0u, 0u};
    }

    float v[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float acc = 0.0f;
        if constexpr (F16) {
            half8 h;
            __builtin_memcpy(&h, &buf[t], 16);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                acc = fmaf(qw[k], (float)h[k], acc);
        } else {
            const float f[4] = {__uint_as_float(buf[t][0]), __uint_as_float(buf[t][1]),
                                __uint_as_float(buf[t][2]), __uint_as_float(buf[t][3])};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc = fmaf(qw[k], f[k], acc);
        }
        v[t] = acc;
    }

    int toff = 0;
    Butterfly<LPR / 2, T>::run(v, lane, toff);

    constexpr int OWN = LPR / T;               // lanes sharing one final sum
    if (lane % OWN != 0)
        return;
    const int64_t r = base + (int64_t)toff * RPL + sub;
    if (r >= a.nb)
        return;
    const float s = v[0];
    if (a.scores)
        a.scores[r] = s;
    if (a.keys || a.hist) {
        const uint32_t key = score_key(s);
        if (a.keys)
            a.keys[r] = key;
        if (a.hist)
            atomicAdd(&a.hist[key >> (32 - kHistBits)], 1u);
    }
}

__global__ __launch_bounds__(256) void k_keys_hist(const float *scores, int32_t nb, uint32_t *keys,
                                                   uint32_t *hist)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nb; i += gridDim.x * 256) {
        const uint32_t key = score_key(scores[i]);
        keys[i] = key;
        atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
    }
}

template <bool F16, int LPR>
hipError_t go(const ScoreArgs &a, hipStream_t s)
{
    constexpr int T = LPR < 16 ? LPR : 16;
    constexpr int rows_per_wg = 4 * T * (kWave / LPR);
    const int grid = (int)((a.nb + rows_per_wg - 1) / rows_per_wg);
    hipLaunchKernelGGL((k_score<F16, LPR>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

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

hipError_t launch_keys_hist(const float *scores, int32_t nb, uint32_t *keys, uint32_t *hist,
                            hipStream_t s)
{
    if (nb <= 0)
        return hipSuccess;
    int grid = (nb + 255) / 256;
    grid = grid > 2048 ? 2048 : grid;
    hipLaunchKernelGGL(k_keys_hist, dim3(grid), dim3(256), 0, s, scores, nb, keys, hist);
    return hipGetLastError();
}

}  // namespace qsa
