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
//
// Outputs (all optional, plain stores, no atomics): fp32 scores; the
// order-preserving 32-bit key of every score; and, for the top-k, each tile's
// T = R/8 largest composite keys (key << 32 | ~block), sorted descending.
//
// Fused stage 1: in a decode step at most one summary row is new.  Workgroup 0
// (dispatched first) appends the token's rows, pools that block, then scores
// the LAST tile -- the one holding the new row -- so the pooling latency hides
// under the stream of the other workgroups.
#include "qsa_pool.h"
#include "qsa_wave.h"

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

// Tile list: the T largest of the R composites in s_c (0 = no row), written
// descending to lists[tile*T ...]; slots past the tile's rows get 0.  Ranks
// are exact because composites are unique and nonzero.  All 256 threads
// work: P = 256/R consecutive threads share an entry, each counting the
// larger composites in 1/P of the tile, summed with DPP quad moves.  Whole
// workgroup calls (uniform control flow: DPP reads neighbouring lanes).
template <int R, int T>
__device__ inline void write_tile_list(const uint64_t *s_c, uint64_t *lists, int tile, int valid_rows)
{
    static_assert(R == 64 || R == 128 || R == 256, "tile rows");
    constexpr int P = 256 / R;
    constexpr int SPAN = R / P;
    const int i = threadIdx.x / P, part = threadIdx.x % P;
    const uint64_t c = s_c[i];
    uint32_t rank = 0;
#pragma unroll 8
    for (int u = 0; u < SPAN; ++u)
        rank += s_c[part * SPAN + u] > c ? 1u : 0u;
    if constexpr (P >= 2)
        rank += wave::dpp<wave::kQuadXor1>(rank);
    if constexpr (P == 4)
        rank += wave::dpp<wave::kQuadXor2>(rank);
    if (part == 0 && c != 0 && rank < (uint32_t)T)
        lists[(size_t)tile * T + rank] = c;
    // the nonzero composites take ranks [0, valid_rows): the rest are empty
    if ((int)threadIdx.x >= valid_rows && threadIdx.x < (unsigned)T)
        lists[(size_t)tile * T + threadIdx.x] = 0;
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int LPR>
struct ScoreShape {
    static constexpr int RPL = kWave / LPR;           // rows per wave-wide load
    static constexpr int T = LPR < 16 ? LPR : 16;     // loads in flight per lane
    static constexpr int RPW = T * RPL;               // rows per wave tile
    static constexpr int R = 4 * RPW;                 // rows per workgroup tile
};

template <bool F16, int LPR>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a)
{
    using S = ScoreShape<LPR>;
    constexpr int EPL = F16 ? 8 : 4;           // elements per 16-byte chunk
    constexpr int RPL = S::RPL, T = S::T, RPW = S::RPW, R = S::R;
    constexpr int ROWB = LPR * 16;             // row bytes
    __shared__ uint64_t s_c[R];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = lane % LPR;
    const int sub = lane / LPR;
    const int tile = blockIdx.x == 0 ? (int)gridDim.x - 1 : (int)blockIdx.x - 1;
    if (blockIdx.x == 0 && a.fuse) {
        if (a.upd.new_idx_row)
            append_rows(a.upd, threadIdx.x, 256);
        if (a.upd.nblk > 0)
            pool_row<F16>(a.upd, a.upd.b0, threadIdx.x);
        __threadfence();   // the pooled row is read back below by this workgroup
        __syncthreads();
    }
    const int64_t base = ((int64_t)tile * 4 + wave) * RPW;

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
    const int local = wave * RPW + toff * RPL + sub;
    const int64_t r = base + (int64_t)toff * RPL + sub;
    if (lane % OWN == 0) {
        uint64_t c = 0;
        if (r < a.nb) {
            const float s = v[0];
            if (a.scores)
                a.scores[r] = s;
            if (a.keys) {
                const uint32_t key = score_key(s);
                a.keys[r] = key;
                c = comp_key(key, (uint32_t)r);
            }
        }
        s_c[local] = c;
    }
    if (a.lists) {
        __syncthreads();
        const int64_t valid = a.nb - (int64_t)tile * R;
        write_tile_list<R, R / kListDiv>(s_c, a.lists, tile, (int)(valid < R ? valid : R));
    }
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
    write_tile_list<kKeysTile, kKeysTile / kListDiv>(s_c, lists, blockIdx.x,
                                                     valid < kKeysTile ? valid : kKeysTile);
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
    (void)f16;
    switch (row_bytes / 16) {
    case 8: return ScoreShape<8>::R;
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
