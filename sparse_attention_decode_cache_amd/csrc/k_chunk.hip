// k_chunk.hip -- a prefill chunk: n_q consecutive tokens of one sequence in
// one call, with results equal to n_q decode steps in a row; its attention
// also serves the batched decode (one unit per sequence).  Query i sits at
// position p = n0 + i; it sees the floor((p + 1) / 4) blocks completed by then
// (the causal block mask), keeps the top k of them and attends to their cells
// and to its own tail [post 10, "QSA indexer"; "incremental pooled-key
// cache（COMMON-004）"; "selected QSA K/V gather（COMMON-005）"].
//
// Launches (after the caller pools the blocks the chunk completes):
//   prep    per query: q_idx scaled by the head weights (score = sum over
//           (h, d) of w_h q_hd khat_hd, one contraction of length H*D), times
//           a power of two that keeps it in f16 range, split into f16 hi + lo
//           and written in the matrix-core operand layout;
//   score   all queries x all blocks as one f16 MFMA GEMM (hi and lo both
//           multiplied: the products are exact in fp32), epilogue: the
//           order-preserving key of each (scaled) score, 0 past the query's
//           blocks;
//   select  one workgroup per query: the exact top-k over its keys, held
//           in LDS (a linear histogram, then the boundary bin ranked);
//   attend  workgroup (query, split, KV head): the attention unit of
//           qsa_unit.h over the split's share of the query's iterations of
//           64 cells, folded into a running (max, sum, acc) in registers;
//           with one split the output is written directly, otherwise a small
//           merge follows.
#include <type_traits>

#include "qsa_attend.h"
#include "qsa_internal.h"
#include "qsa_select.h"
#include "qsa_unit.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

using namespace att;

// ------------------------------------------------------------------ append

__global__ __launch_bounds__(256) void k_chunk_append(ChunkArgs c)
{
    const size_t ni = (size_t)c.n_q * c.idx_row_bytes / 16;
    const size_t nk = (size_t)c.n_q * c.kv_row_bytes / 16;
    uint4 *di = (uint4 *)((char *)c.idx_k + (size_t)c.n0 * c.idx_row_bytes);
    uint4 *dk = (uint4 *)((char *)c.k + (size_t)c.n0 * c.kv_row_bytes);
    uint4 *dv = (uint4 *)((char *)c.v + (size_t)c.n0 * c.kv_row_bytes);
    const uint4 *si = (const uint4 *)c.idx_rows;
    const uint4 *sk = (const uint4 *)c.k_rows;
    const uint4 *sv = (const uint4 *)c.v_rows;
    const size_t total = ni + 2 * nk;
    for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < total; x += (size_t)gridDim.x * 256) {
        if (x < ni)
            di[x] = si[x];
        else if (x < ni + nk)
            dk[x - ni] = sk[x - ni];
        else
            dv[x - ni - nk] = sv[x - ni - nk];
    }
}

// ------------------------------------------------------------------- prep

typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One wave per query (4 per workgroup).  Lane g owns elements 8g .. 8g+7 of
// the H*D contraction.  Output: for query tile qt (16 queries) and k-step ks
// (32 elements), hi then lo, 64 lanes x 8 halves: lane l holds elements
// 32 ks + 8 (l / 16) .. +8 of query 16 qt + l % 16 -- the B operand of
// v_mfma_f32_16x16x32_f16.  Queries past n_q (tile padding) are zero.
__global__ __launch_bounds__(256) void k_chunk_prep(ChunkArgs c)
{
    const int lane = threadIdx.x & 63;
    const int qi = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int QK = c.H * c.D, KS = QK / 32;
    const bool live = lane < QK / 8;
    const bool real = qi < c.n_q;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = 0.0f;
    if (live && real) {
        const int e0 = 8 * lane;
        const float wh = c.w[(size_t)qi * c.H + e0 / c.D];
        const float4 *src = (const float4 *)(c.q_idx + (size_t)qi * QK + e0);
        const float4 u = src[0], v = src[1];
        x[0] = wh * u.x; x[1] = wh * u.y; x[2] = wh * u.z; x[3] = wh * u.w;
        x[4] = wh * v.x; x[5] = wh * v.y; x[6] = wh * v.z; x[7] = wh * v.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        amax = fmaxf(amax, fabsf(x[j]));
    amax = wave::reduce_max_f(amax);
    // 2^s with amax * 2^s in [2^13, 2^14): far from the f16 limit, lo normal
    int ex = 0;
    (void)frexpf(amax, &ex);
    const int sh = (amax > 0.0f && amax < __builtin_inff()) ? 14 - ex : 0;
    if (live) {
        _Float16 hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float y = ldexpf(x[j], sh);
            hi[j] = (_Float16)y;
            lo[j] = (_Float16)(y - (float)hi[j]);
        }
        const int ks = lane / 4, kg = lane % 4;
        const int l = kg * 16 + qi % 16;
        _Float16 *dst = c.qhl + ((((size_t)(qi / 16) * KS + ks) * 2) * 64 + l) * 8;
        __builtin_memcpy(dst, hi, 16);
        __builtin_memcpy(dst + 64 * 8, lo, 16);
    }
    if (lane == 0 && real)
        c.qscale[qi] = ldexpf(1.0f, -sh);
}

// ------------------------------------------------------------------ score

__device__ inline uint32_t chunk_key(float s)
{
    // -0 and +0 compare equal: canonicalise before taking the bits
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSQT = 8;                      // query tiles (16 queries) per LDS stage
constexpr int kSRT = 2;                      // block row tiles (16 blocks) per wave
constexpr int kSBlocks = 4 * kSRT * 16;      // blocks per workgroup (4 waves)

template <int KS>
struct ScShape {
    static constexpr int KC = 2 < KS ? 2 : KS;                            // k-steps per LDS stage
    static constexpr int NST = KS / KC;                                   // stages per query group
    static constexpr int ES = 4;                                          // summary element bytes
};

// The GEMM over fp32 summaries (f16 summaries take k_chunk_score_bs below).
// Workgroup = 128 blocks x every query, 4 waves.  Wave w keeps the A operand
// of its 32 blocks (two 16-row tiles, every k-step, as f16 hi and lo) in
// registers for the whole kernel: the summaries are read once; a query's hi
// and lo halves meet the rows' hi half, its hi half their lo half (the lo x
// lo product is below 2^-22 of the term).
// The queries stream through LDS, 128 queries x KC k-steps per stage, the
// next stage loaded straight into the other LDS buffer while the current one
// runs on the matrix cores; each B fragment read from LDS feeds both row tiles.  After the last
// stage of a query group, the epilogue writes its keys (and, with SCORES,
// the fp32 scores).  The two buffers are two LDS arrays of their own: with
// one array indexed by the buffer, the compiler cannot tell a stage's reads
// from the next stage's direct-to-LDS loads and waits for those loads right
// after issuing them.
template <int KS, bool SCORES>
__global__ __launch_bounds__(256) void k_chunk_score(ChunkArgs c)
{
    using S = ScShape<KS>;
    constexpr int KC = S::KC, NST = S::NST, ES = S::ES;
    __shared__ uint4 sb0[kSQT][KC][2][64];
    __shared__ uint4 sb1[kSQT][KC][2][64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    constexpr int QK = 32 * KS;
    const int QT = (c.n_q + 15) / 16;
    const int nqg = (QT + kSQT - 1) / kSQT;
    const int64_t bw = (int64_t)blockIdx.x * kSBlocks + wave * kSRT * 16;
    const int mr = lane & 15, kg = lane >> 4;

    // A: lane l holds row l % 16 of each row tile, elements 32 ks + 8 (l / 16) .. +8
    half8 ah[kSRT][KS], al[kSRT][KS];
#pragma unroll
    for (int rt = 0; rt < kSRT; ++rt) {
        int64_t r = bw + 16 * rt + mr;
        r = r < c.nb_last ? r : c.nb_last - 1;
        const char *row = (const char *)c.summary + ((size_t)r * QK + 8 * kg) * ES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float f[8];
            const uint4 v0 = *(const uint4 *)(row + (size_t)(32 * ks) * ES);
            const uint4 v1 = *(const uint4 *)(row + (size_t)(32 * ks) * ES + 16);
            __builtin_memcpy(f, &v0, 16);
            __builtin_memcpy(f + 4, &v1, 16);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ah[rt][ks][j] = (_Float16)f[j];
                al[rt][ks][j] = (_Float16)(f[j] - (float)ah[rt][ks][j]);
            }
        }
    }

    // B stages: 128 queries x KC k-steps, 64 segments (ct, kk, hl) of 64
    // 16-byte operand slots, double-buffered in LDS and filled straight from
    // memory (global_load_lds: lane l's 16 bytes land at the segment base +
    // 16 l); wave w issues segments w, w + 4, ...  The query operand buffer is
    // padded with zeros to whole groups of 128 queries.
    const uint4 *qsrc = (const uint4 *)c.qhl;
    constexpr int NSEG = kSQT * KC * 2;
    auto issue_b = [&](int qg, int kc, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NSEG / 4; ++u) {
            const int seg = wave + 4 * u;
            const int hl = seg & 1, kk = (seg >> 1) % KC, ct = (seg >> 1) / KC;
            const int qt = qg * kSQT + ct;
            const uint4 *src = qsrc + (((size_t)qt * KS + kc * KC + kk) * 2 + hl) * 64 + lane;
            uint4 *dst = buf ? &sb1[ct][kk][hl][0] : &sb0[ct][kk][hl][0];
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
        }
    };

    const int nst = nqg * NST;
    issue_b(0, 0, 0);
    for (int qg = 0; qg < nqg; ++qg) {
        float4v acc[kSRT][kSQT];
#pragma unroll
        for (int rt = 0; rt < kSRT; ++rt)
#pragma unroll
            for (int ct = 0; ct < kSQT; ++ct)
                acc[rt][ct] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kc = 0; kc < NST; ++kc) {
            const int gs = qg * NST + kc, buf = gs & 1;
            // this stage's segments (every wave's) have landed, and every
            // wave is done with the other buffer (read in stage gs - 1)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (gs + 1 < nst)
                issue_b(kc + 1 < NST ? qg : qg + 1, kc + 1 < NST ? kc + 1 : 0, buf ^ 1);
            // fragments f = (kk, hl, ct) in this order, read from LDS FD
            // ahead of their two MFMAs (both row tiles); the order is pinned so
            // that the reads stay ahead, and a tile's hi and lo products are
            // 16 MFMAs apart
            constexpr int NF = KC * 2 * kSQT, FD = 4;
            auto frag = [&](int f) __attribute__((always_inline)) -> half8 {
                const int ct = f % kSQT, hl = (f / kSQT) & 1, kk = f / (2 * kSQT);
                half8 x;
                __builtin_memcpy(&x, buf ? &sb1[ct][kk][hl][lane] : &sb0[ct][kk][hl][lane], 16);
                return x;
            };
            half8 fr[FD];
#pragma unroll
            for (int f = 0; f < FD; ++f)
                fr[f] = frag(f);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int ct = f % kSQT, hl = (f / kSQT) & 1, ks = kc * KC + f / (2 * kSQT);
#pragma unroll
                for (int rt = 0; rt < kSRT; ++rt)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][ks], fr[f % FD], acc[rt][ct], 0, 0, 0);
                if (hl == 0) {
#pragma unroll
                    for (int rt = 0; rt < kSRT; ++rt)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rt][ks], fr[f % FD], acc[rt][ct], 0, 0, 0);
                }
                if (f + FD < NF)
                    fr[f % FD] = frag(f + FD);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // lane l holds D[block 4 (l / 16) + j][query l % 16] of each tile.
        // The keys are taken on the scaled sums: a query's keys are compared
        // only with each other, and its power-of-two factor is exact, so it
        // changes neither their order nor their ties; only the optional fp32
        // scores are scaled back.
#pragma unroll
        for (int ct = 0; ct < kSQT; ++ct) {
            const int qi = (qg * kSQT + ct) * 16 + mr;
            if (qi >= c.n_q)
                continue;
            const int64_t nbq = ((int64_t)c.n0 + qi + 1) >> 2;
#pragma unroll
            for (int rt = 0; rt < kSRT; ++rt) {
                const int64_t b = bw + 16 * rt + 4 * kg;
                u32x4 key;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    key[j] = b + j < nbq ? chunk_key(acc[rt][ct][j]) : 0u;
                if (b < c.ldk)
                    *(u32x4 *)(c.keys + (size_t)qi * c.ldk + b) = key;
            }
            if constexpr (SCORES) {
                const float f = c.qscale[qi];
#pragma unroll
                for (int rt = 0; rt < kSRT; ++rt) {
                    const int64_t b = bw + 16 * rt + 4 * kg;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (b + j < c.nb_last)
                            c.scores_out[(size_t)qi * c.nb_last + b + j] =
                                b + j < nbq ? acc[rt][ct][j] * f : -INFINITY;
                }
            }
        }
    }
}

// The f16 summaries' GEMM with the roles turned round: each wave keeps ONE
// tile of 16 queries (f16 hi and lo, every k-step) in registers for the whole
// kernel, and the blocks stream past it.  Workgroup = 8 waves = 128 queries x
// one range of row tiles.  The range's rows go through LDS in stages of 32 KB
// (RT = 32 / KS tiles of 16 rows): each stage is loaded into registers
// kBsAhead steps before it is due, written to one of two LDS buffers in the
// step before, and read there by every wave; every summary fragment read
// from LDS feeds two products (the query's hi and lo).  Chunk c of row r of
// a stage sits at slot c ^ (r % 16) of the row: the 16 rows that one
// fragment read takes at one chunk position then fall in distinct banks, and
// each load still covers whole rows.  The workgroups of one row range (its
// query groups) are numbered so that they run on one XCD (dispatch deals
// workgroups to the XCDs in turn) and read the range once into its L2.
constexpr int kBsWaves = 8;                  // query tiles per workgroup
constexpr int kBsAhead = 4;                  // steps between a stage's loads and its use
constexpr int kBsStage = 32 * 1024;          // bytes per stage
constexpr size_t kBsLds = 2 * (size_t)kBsStage;
constexpr int kXcds = 8;

template <int KS>
struct BsShape {
    static constexpr int RB = 64 * KS;                       // row bytes (f16)
    static constexpr int CPR = 4 * KS;                       // 16-byte chunks per row
    static constexpr int RT = kBsStage / (16 * RB);          // row tiles per stage
    static constexpr int SEG = kBsStage / 1024 / kBsWaves;   // 16-byte pieces per lane per stage
    static_assert(RT >= 1 && RT * 16 * RB == kBsStage, "a stage is whole row tiles");
};

template <int KS, bool SCORES>
__global__ __launch_bounds__(64 * kBsWaves) void k_chunk_score_bs(ChunkArgs c, int32_t n_qg, int32_t tiles_per)
{
    using S = BsShape<KS>;
    constexpr int RT = S::RT, CPR = S::CPR, SEG = S::SEG;
    constexpr int NV = kBsStage / 16;
    static_assert(kBsAhead == 4, "the step loop below is unrolled by four");
    extern __shared__ uint4 ring[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int nwg = (int)gridDim.x;            // a multiple of kXcds
    const int lin = ((int)blockIdx.x % kXcds) * (nwg / kXcds) + (int)blockIdx.x / kXcds;
    const int ms = lin / n_qg, qg = lin % n_qg;
    const int mt = (c.nb_last + 15) / 16;
    const int tile0 = ms * tiles_per;
    const int tile1 = tile0 + tiles_per < mt ? tile0 + tiles_per : mt;
    if (tile0 >= tile1)
        return;
    const int nst = (tile1 - tile0 + RT - 1) / RT;
    // whole groups of kBsAhead steps, so that no load or LDS write in the
    // loop is conditional and the compiler's count of loads in flight stays
    // exact around it; the stages past nst load rows past the range (held to
    // the last row at the end of the summaries) and store nothing
    const int nstp = (nst + kBsAhead - 1) / kBsAhead * kBsAhead;
    const int qt = qg * kBsWaves + wave;
    const int qi = qt * 16 + (lane & 15);
    const int kg = lane >> 4;

    // B: this wave's query tile (padded with zeros to whole groups of 8 tiles)
    half8 bh[KS], bl[KS];
    {
        const uint4 *qsrc = (const uint4 *)c.qhl + (size_t)qt * KS * 2 * 64 + lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 h = qsrc[(2 * ks) * 64], l = qsrc[(2 * ks + 1) * 64];
            __builtin_memcpy(&bh[ks], &h, 16);
            __builtin_memcpy(&bl[ks], &l, 16);
        }
    }
    const bool live = qi < c.n_q;
    const int64_t nbq = ((int64_t)c.n0 + qi + 1) >> 2;
    const float qs = SCORES && live ? c.qscale[qi] : 1.0f;

    const char *rows = (const char *)c.summary;
    const int64_t last = c.nb_last - 1;
    // this lane's SEG pieces of stage j (slot f = 64 seg + lane of the stage)
    auto load = [&](int j, u32x4 *dst) __attribute__((always_inline)) {
        const int64_t r0 = (int64_t)(tile0 + j * RT) * 16;
#pragma unroll
        for (int u = 0; u < SEG; ++u) {
            const int f = (wave + kBsWaves * u) * 64 + lane;
            const int rr = f / CPR, slot = f % CPR;
            const int chunk = slot ^ (rr & 15 & (CPR - 1));
            int64_t r = r0 + rr;
            r = r < last ? r : last;
            dst[u] = *((const u32x4 *)(rows + r * S::RB) + chunk);
        }
    };
    auto put = [&](int j, const u32x4 *src) __attribute__((always_inline)) {
        u32x4 *buf = (u32x4 *)(ring + (j & 1) * NV);
#pragma unroll
        for (int u = 0; u < SEG; ++u)
            buf[(wave + kBsWaves * u) * 64 + lane] = src[u];
    };
    // fragment (rt, ks = 4 m + n) of this lane: row r = lane % 16, chunk
    // 4 ks + kg, stored at slot 16 m + ((4 n + kg) ^ r) of the row: four
    // per-lane offsets, the rest immediate
    int sidx[4];
    {
        const int r = lane & 15, rx = r & (CPR - 1) & 15;
#pragma unroll
        for (int n = 0; n < 4; ++n)
            sidx[n] = r * CPR + ((4 * n + kg) ^ rx);
    }
    auto run = [&](int st) __attribute__((always_inline)) {
        const uint4 *buf = ring + (st & 1) * NV;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            half8 a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                __builtin_memcpy(&a[ks], &buf[rt * 16 * CPR + 16 * (ks / 4) + sidx[ks % 4]], 16);
            float4v ach = {0.0f, 0.0f, 0.0f, 0.0f}, acl = ach;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ach = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], bh[ks], ach, 0, 0, 0);
                acl = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], bl[ks], acl, 0, 0, 0);
            }
            // lane l holds D[block 4 (l / 16) + j][query l % 16]; keys on the
            // scaled sums (a query's power of two changes no order or tie)
            const int tile = tile0 + st * RT + rt;
            const int64_t b = (int64_t)tile * 16 + 4 * kg;
            if (tile < tile1 && live) {
                u32x4 key;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    key[j] = b + j < nbq ? chunk_key(ach[j] + acl[j]) : 0u;
                if (b < c.ldk)
                    *(u32x4 *)(c.keys + (size_t)qi * c.ldk + b) = key;
                if constexpr (SCORES) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (b + j < c.nb_last)
                            c.scores_out[(size_t)qi * c.nb_last + b + j] =
                                b + j < nbq ? (ach[j] + acl[j]) * qs : -INFINITY;
                }
            }
        }
    };
    // step st: after the barrier (fenced for LDS only) stage st is in its
    // buffer and every wave is done with stage st - 1, whose buffer stage
    // st + 1 then takes; the registers that held stage st load st + 4
    auto step = [&](int st, u32x4 *mine, const u32x4 *next) __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        load(st + kBsAhead, mine);
        put(st + 1, next);
        run(st);
    };
    u32x4 r0[SEG], r1[SEG], r2[SEG], r3[SEG];
    load(0, r0);
    load(1, r1);
    load(2, r2);
    load(3, r3);
    put(0, r0);
    for (int s0 = 0; s0 < nstp; s0 += kBsAhead) {
        step(s0, r0, r1);
        step(s0 + 1, r1, r2);
        step(s0 + 2, r2, r3);
        step(s0 + 3, r3, r0);
    }
}

template <int KS>
hipError_t score_go(const ChunkArgs &c, dim3 grid, hipStream_t s)
{
    if (c.scores_out)
        hipLaunchKernelGGL((k_chunk_score<KS, true>), grid, dim3(256), 0, s, c);
    else
        hipLaunchKernelGGL((k_chunk_score<KS, false>), grid, dim3(256), 0, s, c);
    return hipGetLastError();
}

// f16 summaries: the query-stationary GEMM, one workgroup per CU (256 in
// all, 8 waves each), row ranges split evenly over the query groups' share.
template <int KS>
hipError_t score_bs_go(const ChunkArgs &c, hipStream_t s)
{
    static_assert(kBsWaves == kSQT, "the prep pads the queries to whole groups of 8 tiles");
    const int qt = (c.n_q + 15) / 16;
    const int n_qg = (qt + kBsWaves - 1) / kBsWaves;
    const int mt = (int)((c.nb_last + 15) / 16);
    int n_ms = (256 + n_qg - 1) / n_qg;
    n_ms = n_ms < mt ? n_ms : mt;
    // ranges of whole groups of kBsAhead stages (the kernel pads to them)
    constexpr int q = kBsAhead * BsShape<KS>::RT;
    const int tiles_per = ((mt + n_ms - 1) / n_ms + q - 1) / q * q;
    n_ms = (mt + tiles_per - 1) / tiles_per;
    const int nwg = (n_qg * n_ms + kXcds - 1) / kXcds * kXcds;
    if (c.scores_out)
        hipLaunchKernelGGL((k_chunk_score_bs<KS, true>), dim3(nwg), dim3(64 * kBsWaves), kBsLds, s, c, n_qg, tiles_per);
    else
        hipLaunchKernelGGL((k_chunk_score_bs<KS, false>), dim3(nwg), dim3(64 * kBsWaves), kBsLds, s, c, n_qg, tiles_per);
    return hipGetLastError();
}

template <bool F16>
hipError_t score_ks(const ChunkArgs &c, dim3 grid, hipStream_t s)
{
    if constexpr (F16) {
        switch (c.H * c.D / 32) {
        case 2: return score_bs_go<2>(c, s);
        case 4: return score_bs_go<4>(c, s);
        case 8: return score_bs_go<8>(c, s);
        case 16: return score_bs_go<16>(c, s);
        }
    } else {
        switch (c.H * c.D / 32) {   // fp32 rows are at most 1 KB: 256 elements
        case 2: return score_go<2>(c, grid, s);
        case 4: return score_go<4>(c, grid, s);
        case 8: return score_go<8>(c, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- select

// The chunk select's LDS is Smem, the id bitmap and a list of up to
// kChunkKeep composites: its passes read a query's keys from memory (L2)
// rather than holding them all in LDS, so that two of its workgroups share a
// CU and hide each other's latency (with the keys held, one per CU: 66
// against 59 us at 1024 queries x 31,819 blocks); the keys above the pruning
// bound (a few per cent) are listed by the histogram pass, so the marking
// pass reads the list instead of memory.
constexpr uint32_t kChunkKeep = 4096;

__host__ __device__ inline size_t chunk_sel_lds(int32_t nb)
{
    return sel::lds_bytes(nb) + sizeof(uint64_t) * kChunkKeep;
}

__global__ __launch_bounds__(sel::kT) void k_chunk_select(ChunkArgs c)
{
    extern __shared__ uint4 sel_lds[];
    const int i = blockIdx.x, t = threadIdx.x;
    const int32_t nbq = (int32_t)(((int64_t)c.n0 + i + 1) >> 2);
    const int32_t keep = nbq < c.kb ? nbq : c.kb;
    int32_t *row_out = c.sel_out ? c.sel_out + (size_t)i * c.kb : nullptr;
    if (row_out)
        for (int j = keep + t; j < c.kb; j += sel::kT)
            row_out[j] = -1;
    if (nbq <= c.kb) {
        if (row_out)
            for (int j = t; j < nbq; j += sel::kT)
                row_out[j] = j;
        return;
    }
    SelectArgs a{};
    a.keys = c.keys + (size_t)i * c.ldk;
    a.nb = nbq;
    a.k = c.kb;
    a.T = 8;
    int32_t *row = c.sel + (size_t)i * c.kb;
    char *lds = reinterpret_cast<char *>(sel_lds);
    sel::Smem &sm = *reinterpret_cast<sel::Smem *>(lds);
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(lds + (sizeof(sel::Smem) + 15) / 16 * 16);
    uint32_t *lkeys = nullptr;
    uint64_t *klist = reinterpret_cast<uint64_t *>(lds + sel::lds_bytes(nbq));
    sel::keys_path(a, sm, bitmap, lkeys, [=](uint32_t slot, uint32_t id) {
        row[slot] = (int32_t)id;
        if (row_out)
            row_out[slot] = (int32_t)id;
    }, klist, kChunkKeep);
}

// ----------------------------------------------------------------- attend
//
// Workgroup (query, split, KV head), 512 threads (two workgroups per CU, so
// that one computes while the other waits): the attention unit of
// qsa_unit.h over the split's 64-cell iterations.

constexpr int kCAT = 512;                    // threads (two workgroups share a CU)
using unit::CALds;
using unit::QueryUnit;
using unit::kCI;

template <int DH, int G>
__global__ __launch_bounds__(kCAT, 2) void k_chunk_attend(ChunkArgs c)
{
    extern __shared__ uint4 ca_lds[];
    CALds<DH, G> &L = *reinterpret_cast<CALds<DH, G> *>(ca_lds);
    const int ns = c.n_split;
    const int i = blockIdx.x / ns;
    QueryUnit u{};
    u.k = c.k;
    u.v = c.v;
    u.sel = c.sel + (size_t)i * c.kb;
    u.q = c.q + (size_t)i * c.kv_heads * G * DH;
    u.out = c.out + (size_t)i * c.kv_heads * G * DH;
    u.part = c.part + (size_t)i * c.kv_heads * ns * part_stride(G, DH);
    u.n = (int64_t)c.n0 + i + 1;
    u.kb = c.kb;
    u.kv_heads = c.kv_heads;
    u.ns = ns;
    u.direct = ns == 1;
    u.scale = c.scale;
    unit::attend_unit<DH, G, kCAT, unit::kSplits>(u, L, blockIdx.x % ns, blockIdx.y);
}

// Batched decode: workgroups [wg0[s], wg0[s+1]) are sequence s's (split, KV
// head) units.
template <int DH, int G>
__global__ __launch_bounds__(kCAT, 2) void k_batch_attend(AttendBatchArgs b)
{
    extern __shared__ uint4 ca_lds[];
    CALds<DH, G> &L = *reinterpret_cast<CALds<DH, G> *>(ca_lds);
    int sq = 0;
    while (sq + 1 < b.n && (int)blockIdx.x >= b.wg0[sq + 1])
        ++sq;
    const AttendArgs &a = b.seq[sq];
    const int local = (int)blockIdx.x - b.wg0[sq];
    QueryUnit u{};
    u.k = a.k;
    u.v = a.v;
    u.sel = a.sel;
    u.q = a.q;
    u.out = a.out;
    u.part = a.part;
    u.n = 4 * (int64_t)a.nb + (a.n_cells - 4 * (int64_t)a.n_sel_blocks);
    u.kb = a.n_sel_blocks;
    u.kv_heads = a.kv_heads;
    u.ns = a.n_split;
    u.direct = 0;                                  // the merge kernel writes the output
    u.scale = a.scale;
    unit::attend_unit<DH, G, kCAT, unit::kSplits>(u, L, local % a.n_split, local / a.n_split);
}

// The selection as a bitmap over the blocks (bit b of word b / 32): one
// thread per word finds its first id by binary search in the ascending ids.
__global__ __launch_bounds__(256) void k_sel_bitmap(const int32_t *sel, int32_t n_sel, int32_t nb,
                                                    uint32_t *bitmap)
{
    const int32_t wd = blockIdx.x * 256 + threadIdx.x;
    if (wd >= (nb + 31) / 32)
        return;
    const int32_t lo_id = 32 * wd;
    int32_t lo = 0, hi = n_sel;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (sel[mid] < lo_id)
            lo = mid + 1;
        else
            hi = mid;
    }
    uint32_t bits = 0;
    for (int32_t i = lo; i < n_sel && sel[i] < lo_id + 32; ++i)
        bits |= 1u << (sel[i] - lo_id);
    bitmap[wd] = bits;
}

template <int DH, int G>
__global__ __launch_bounds__(kCAT, 2) void k_masked_attend(MaskedArgs m)
{
    extern __shared__ uint4 ca_lds[];
    CALds<DH, G> &L = *reinterpret_cast<CALds<DH, G> *>(ca_lds);
    QueryUnit u{};
    u.k = m.k;
    u.v = m.v;
    u.sel = nullptr;
    u.q = m.q;
    u.out = m.out;
    u.part = m.part;
    u.n = m.n_tokens;
    u.kb = (int32_t)(m.n_tokens / 4);
    u.kv_heads = m.kv_heads;
    u.ns = m.n_split;
    u.direct = m.n_split == 1;
    u.scale = m.scale;
    u.mask = m.bitmap;
    unit::attend_unit<DH, G, kCAT, unit::kMasked>(u, L, blockIdx.x, blockIdx.y);
}

template <int DH, int G>
hipError_t masked_go(const MaskedArgs &m, hipStream_t s)
{
    const size_t lds = sizeof(CALds<DH, G>);
    if (lds > 64 * 1024) {
        static hipError_t attr = hipFuncSetAttribute((const void *)k_masked_attend<DH, G>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL((k_masked_attend<DH, G>), dim3(m.n_split, m.kv_heads), dim3(kCAT), lds, s, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || m.n_split == 1)
        return e;
    return launch_merge_chunk(m.part, m.out, 1, m.kv_heads, m.n_split, DH, G, s);
}

template <int DH, int G>
hipError_t attend_go(const ChunkArgs &c, hipStream_t s)
{
    const size_t lds = sizeof(CALds<DH, G>);
    if (lds > 64 * 1024) {
        static hipError_t attr = hipFuncSetAttribute((const void *)k_chunk_attend<DH, G>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL((k_chunk_attend<DH, G>), dim3(c.n_q * c.n_split, c.kv_heads), dim3(kCAT), lds, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.n_split == 1)
        return e;
    return launch_merge_chunk(c.part, c.out, c.n_q, c.kv_heads, c.n_split, DH, G, s);
}

template <int DH, int G>
hipError_t batch_go(AttendBatchArgs &b, hipStream_t s)
{
    b.wg0[0] = 0;
    for (int i = 0; i < b.n; ++i) {
        AttendArgs &a = b.seq[i];
        if (a.kv_heads != b.seq[0].kv_heads || a.n_cells < 1)
            return hipErrorInvalidValue;
        // one 64-cell iteration per workgroup: the batch fills the chip
        const int nit = (a.n_cells + kCI - 1) / kCI;
        a.n_split = nit < kChunkMaxSplits ? nit : kChunkMaxSplits;
        b.wg0[i + 1] = b.wg0[i] + a.n_split * a.kv_heads;
    }
    const size_t lds = sizeof(CALds<DH, G>);
    if (lds > 64 * 1024) {
        static hipError_t attr = hipFuncSetAttribute((const void *)k_batch_attend<DH, G>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL((k_batch_attend<DH, G>), dim3(b.wg0[b.n]), dim3(kCAT), lds, s, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // sequences kept in one split still take the merge (it divides by l)
    return launch_merge_batch(b, DH, G, s);
}

template <int DH>
hipError_t attend_g(const ChunkArgs &c, int G, hipStream_t s)
{
    switch (G) {
    case 1: return attend_go<DH, 1>(c, s);
    case 2: return attend_go<DH, 2>(c, s);
    case 4: return attend_go<DH, 4>(c, s);
    case 8: return attend_go<DH, 8>(c, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend_batch(AttendBatchArgs &b, int Dh, int G, hipStream_t s)
{
    if (b.n < 1 || b.n > kMaxBatch)
        return hipErrorInvalidValue;
#define QSA_BATCH_G(DHV)                                   \
    switch (G) {                                           \
    case 1: return batch_go<DHV, 1>(b, s);                 \
    case 2: return batch_go<DHV, 2>(b, s);                 \
    case 4: return batch_go<DHV, 4>(b, s);                 \
    case 8: return batch_go<DHV, 8>(b, s);                 \
    }                                                      \
    return hipErrorInvalidValue;
    switch (Dh) {
    case 64: QSA_BATCH_G(64)
    case 128: QSA_BATCH_G(128)
    case 256: QSA_BATCH_G(256)
    }
#undef QSA_BATCH_G
    return hipErrorInvalidValue;
}

hipError_t launch_masked_attend(MaskedArgs m, int Dh, int G, hipStream_t s)
{
    const int32_t nb = (int32_t)(m.n_tokens / 4);
    const int32_t nit = (int32_t)((m.n_tokens + kCI - 1) / kCI);
    // enough splits to fill the chip twice over (two workgroups per CU), each
    // holding whole iterations and at most kChunkMaxIds block ids
    int32_t ns = nit < kMaskedSplits ? nit : kMaskedSplits;
    while ((int64_t)((nit + ns - 1) / ns) * (kCI / 4) > kChunkMaxIds)
        ++ns;
    if (ns > kMaskedMaxSplits)
        return hipErrorInvalidValue;
    m.n_split = ns;
    if (nb > 0) {
        const int words = (nb + 31) / 32;
        hipLaunchKernelGGL(k_sel_bitmap, dim3((words + 255) / 256), dim3(256), 0, s, m.sel,
                           m.n_sel_blocks, nb, m.bitmap);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
#define QSA_MASKED_G(DHV)                          \
    switch (G) {                                   \
    case 1: return masked_go<DHV, 1>(m, s);        \
    case 2: return masked_go<DHV, 2>(m, s);        \
    case 4: return masked_go<DHV, 4>(m, s);        \
    case 8: return masked_go<DHV, 8>(m, s);        \
    }                                              \
    return hipErrorInvalidValue;
    switch (Dh) {
    case 64: QSA_MASKED_G(64)
    case 128: QSA_MASKED_G(128)
    case 256: QSA_MASKED_G(256)
    }
#undef QSA_MASKED_G
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_append(const ChunkArgs &c, hipStream_t s)
{
    if (c.idx_row_bytes % 16 || c.kv_row_bytes % 16)
        return hipErrorInvalidValue;
    const size_t total = (size_t)c.n_q * (c.idx_row_bytes + 2 * (size_t)c.kv_row_bytes) / 16;
    size_t grid = (total + 255) / 256;
    grid = grid < 1 ? 1 : (grid > 2048 ? 2048 : grid);
    hipLaunchKernelGGL(k_chunk_append, dim3((unsigned)grid), dim3(256), 0, s, c);
    return hipGetLastError();
}

hipError_t launch_chunk_rest(ChunkArgs c, bool f16, int Dh, int G, hipStream_t s)
{
    const int QK = c.H * c.D;
    if (QK % 32 || QK / 8 > 64 || c.kb < 1 || c.kb >= kChunkMaxIds || c.n_split < 1 ||
        c.n_split > kChunkMaxSplits || c.n_q < 1)
        return hipErrorInvalidValue;
    hipError_t e;
    // scoring and selection only when some query has more blocks than it keeps
    if (c.nb_last > c.kb) {
        // query tiles padded to whole groups of kSQT (zero-filled by the prep)
        const int qt = (c.n_q + 15) / 16;
        const int qt_pad = (qt + kSQT - 1) / kSQT * kSQT;
        hipLaunchKernelGGL(k_chunk_prep, dim3(qt_pad * 4), dim3(256), 0, s, c);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        const dim3 grid((unsigned)((c.nb_last + kSBlocks - 1) / kSBlocks));
        e = f16 ? score_ks<true>(c, grid, s) : score_ks<false>(c, grid, s);
        if (e != hipSuccess)
            return e;
    }
    if (c.nb_last > c.kb || c.sel_out) {
        const size_t lds = chunk_sel_lds(c.nb_last);
        if (lds > sel::kMaxLds)
            return hipErrorInvalidValue;
        if (lds > 64 * 1024) {
            static hipError_t attr = hipFuncSetAttribute((const void *)k_chunk_select,
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         (int)sel::kMaxLds);
            if (attr != hipSuccess)
                return attr;
        }
        hipLaunchKernelGGL(k_chunk_select, dim3(c.n_q), dim3(sel::kT), lds, s, c);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    if (c.union_q > 0)
        return launch_union(c, Dh, G, s);
    switch (Dh) {
    case 64: return attend_g<64>(c, G, s);
    case 128: return attend_g<128>(c, G, s);
    case 256: return attend_g<256>(c, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace qsa
