// k_attend.hip -- stage 4: attention over the gathered cells only.
//
// [post 10, "selected QSA K/V gather（COMMON-005）"]: only the K/V rows of the
// chosen cells (4 per chosen block, plus the tail of the unfinished block) are
// read, and ordinary softmax attention runs over them.  Here the gather is not
// materialised: the attention workgroups load the selected rows directly.
//
// Split-context flash decode.  Cells are enumerated e = 0..n_cells-1 (chosen
// blocks ascending, 4 cells each, then the tail).  Workgroup (split, g) takes
// C = 16 (Dh >= 128) or 32 (Dh = 64) consecutive cells of KV head g -- about
// 258 workgroups for 2051 cells and 2 KV heads, so the whole chip loads in
// parallel -- for all G query heads of that
// group (GQA: each K/V row is read once for G heads).  Per wave, one lane
// covers 8 dims of a cell (Dh/8 lanes per cell), so a wave-wide 16-byte load
// brings whole rows.  All K and V loads of a lane are issued up front.
//   QK:  per-lane partial dots for G heads, transposing butterfly over the
//        Dh/8 lanes of the cell -> logits in LDS;
//   softmax over the split's cells, per head (one wave reduction);
//   PV:  per-lane accumulation, butterfly across the cells of a wave, LDS sum
//        across the 4 waves -> partial (m, l, acc) in the workspace.
// A second kernel merges the partials of a head in split order (fixed order:
// bitwise repeatable).
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

template <int O, int CNT>
struct Butterfly {
    // Before: v[0..CNT) partial sums of CNT different outputs.  Exchanges over
    // lane offsets O, O/2, ..., STOP (exclusive) halve the live set each round.
    template <int STOP>
    static __device__ inline void run(float *v, int lane, int &toff)
    {
        if constexpr (O <= STOP) {
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
            Butterfly<O / 2, H>::template run<STOP>(v, lane, toff);
        } else {
            v[0] += __shfl_xor(v[0], O);
            Butterfly<O / 2, 1>::template run<STOP>(v, lane, toff);
        }
    }
};

__device__ inline float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

template <int DH, int G>
__global__ __launch_bounds__(256) void k_attend(AttendArgs a)
{
    constexpr int LPC = DH / 8;                 // lanes per cell
    constexpr int CPL = kWave / LPC;            // cells per wave-wide load
    constexpr int CPW = cells_per_split(DH);    // cells per workgroup
    constexpr int CPWW = CPW / 4;               // cells per wave
    constexpr int IT = CPWW / CPL;              // loads per lane (each of K and V)
    static_assert(IT >= 1 && G <= LPC && G * 8 >= CPL, "unsupported attention shape");

    __shared__ float s_lg[CPW][G];
    __shared__ float s_m[G], s_l[G];
    __shared__ float s_red[4][G][DH];

    __shared__ int32_t s_blk[CPW / 4];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int sub = lane / LPC;                 // cell within a wave-wide load
    const int chunk = lane % LPC;               // dims [8*chunk, 8*chunk + 8)
    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int e0 = split * CPW;

    // The split's chosen block ids, staged once so that the K/V addresses
    // below need no dependent global load.
    if (a.sel && t < CPW / 4) {
        const int i = e0 / 4 + t;
        s_blk[t] = i < a.n_sel_blocks ? a.sel[i] : -1;
    }
    __syncthreads();

    // Every K and V load of this lane, issued back to back.  Cells outside
    // the list (or with an id outside [0, nb)) read row 0 and are masked.
    uint4 kr[IT], vr[IT];
    bool ok[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int lc = wave * CPWW + it * CPL + sub;
        const int e = e0 + lc;
        bool v = e < a.n_cells;
        int64_t cell = e;
        if (a.sel) {
            if (e < 4 * a.n_sel_blocks) {
                const int32_t b = s_blk[lc >> 2];
                v = v && (uint32_t)b < (uint32_t)a.nb;
                cell = 4 * (int64_t)b + (e & 3);
            } else {
                cell = 4 * (int64_t)a.nb + (e - 4 * a.n_sel_blocks);
            }
        }
        ok[it] = v;
        const size_t off = ((size_t)(v ? cell : 0) * a.kv_heads + g) * DH + (size_t)chunk * 8;
        kr[it] = *(const uint4 *)(a.k + off);
        vr[it] = *(const uint4 *)(a.v + off);
    }

    float qr[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4 *qp = (const float4 *)(a.q + (size_t)(g * G + h) * DH + chunk * 8);
        const float4 x = qp[0], y = qp[1];
        qr[h][0] = x.x; qr[h][1] = x.y; qr[h][2] = x.z; qr[h][3] = x.w;
        qr[h][4] = y.x; qr[h][5] = y.y; qr[h][6] = y.z; qr[h][7] = y.w;
    }

    // ---- logits
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        half8 kh;
        __builtin_memcpy(&kh, &kr[it], 16);
        float kf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kf[j] = (float)kh[j];
        float p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc = fmaf(qr[h][j], kf[j], acc);
            p[h] = acc;
        }
        int hoff = 0;
        Butterfly<LPC / 2, G>::template run<0>(p, lane, hoff);
        constexpr int OWN = LPC / G;
        if (chunk % OWN == 0) {
            const int lc = wave * CPWW + it * CPL + sub;
            s_lg[lc][hoff] = ok[it] ? a.scale * p[0] : -INFINITY;
        }
    }
    __syncthreads();

    // ---- softmax over the split's cells, one head per wave at a time
    static_assert(CPW <= kWave, "one cell per lane in the softmax");
    for (int h = wave; h < G; h += 4) {
        const float x = lane < CPW ? s_lg[lane][h] : -INFINITY;
        const float m = wave_max(x);             // -inf only if no cell of the split is valid
        const float p = x == -INFINITY ? 0.0f : expf(x - m);
        const float l = wave_sum(p);
        if (lane < CPW)
            s_lg[lane][h] = p;
        if (lane == 0) {
            s_m[h] = m;
            s_l[h] = l;
        }
    }
    __syncthreads();

    // ---- P . V
    float acc[G * 8];
#pragma unroll
    for (int i = 0; i < G * 8; ++i)
        acc[i] = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int lc = wave * CPWW + it * CPL + sub;
        half8 vh;
        __builtin_memcpy(&vh, &vr[it], 16);
        float vf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vf[j] = (float)vh[j];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = s_lg[lc][h];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[h * 8 + j] = fmaf(p, vf[j], acc[h * 8 + j]);
        }
    }
    // Sum over the CPL cells of a wave-wide load: lanes differing in bits >= log2(LPC).
    int ioff = 0;
    Butterfly<32, G * 8>::template run<LPC / 2>(acc, lane, ioff);
    constexpr int LIVE = (G * 8) / CPL;
#pragma unroll
    for (int i = 0; i < LIVE; ++i) {
        const int flat = ioff + i;
        s_red[wave][flat >> 3][chunk * 8 + (flat & 7)] = acc[i];
    }
    __syncthreads();

    float *part = a.part + ((size_t)g * a.n_split + split) * (size_t)part_stride(G, DH);
    for (int i = t; i < G * DH; i += 256) {
        const int h = i / DH, d = i % DH;
        part[2 * G + i] = s_red[0][h][d] + s_red[1][h][d] + s_red[2][h][d] + s_red[3][h][d];
    }
    if (t < G) {
        part[t] = s_m[t];
        part[G + t] = s_l[t];
    }
}

// out[h][d] = sum_s e^(m_s - M) acc_s[h][d] / sum_s e^(m_s - M) l_s.
// Workgroup (h, 64-dim slice): the split weights go to LDS once, then 4 groups
// of 64 threads each stream every 4th split's partials for their dim (many
// independent loads in flight) and are summed in a fixed order, so the result
// is bitwise repeatable.
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 64;
constexpr int kMaxSplits = 1024;

__device__ inline float block_reduce(float v, float *s_tmp, bool is_max)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float y = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, y) : v + y;
    }
    if ((t & 63) == 0)
        s_tmp[t >> 6] = v;
    __syncthreads();
    float r = s_tmp[0];
    for (int i = 1; i < kMergeThreads / 64; ++i)
        r = is_max ? fmaxf(r, s_tmp[i]) : r + s_tmp[i];
    __syncthreads();
    return r;
}

template <int DH, int G>
__global__ __launch_bounds__(kMergeThreads) void k_merge(AttendArgs a)
{
    __shared__ float s_f[kMaxSplits];
    __shared__ float s_tmp[kMergeThreads / 64];
    __shared__ float s_acc[kMergeThreads / kMergeDims][kMergeDims];
    const int h = blockIdx.x;
    const int g = h / G, hh = h % G;
    const int t = threadIdx.x;
    const int ns = a.n_split;
    const size_t ps = (size_t)part_stride(G, DH);
    const float *base = a.part + (size_t)g * ns * ps;

    float mx = -INFINITY;
    for (int s = t; s < ns; s += kMergeThreads) {
        s_f[s] = base[s * ps + hh];
        mx = fmaxf(mx, s_f[s]);
    }
    const float M = block_reduce(mx, s_tmp, true);
    float lsum = 0.0f;
    for (int s = t; s < ns; s += kMergeThreads) {
        const float f = s_f[s] == -INFINITY ? 0.0f : expf(s_f[s] - M);
        s_f[s] = f;
        lsum += f * base[s * ps + G + hh];
    }
    const float L = block_reduce(lsum, s_tmp, false);   // also orders the s_f writes

    constexpr int NG = kMergeThreads / kMergeDims;       // split groups
    const int grp = t / kMergeDims;
    const int d = blockIdx.y * kMergeDims + t % kMergeDims;
    const float *p = base + 2 * G + hh * DH + d;
    float acc = 0.0f;
    int s = grp;
    for (; s + 7 * NG < ns; s += 8 * NG) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            x[i] = p[(size_t)(s + i * NG) * ps];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc = fmaf(s_f[s + i * NG], x[i], acc);
    }
    for (; s < ns; s += NG)
        acc = fmaf(s_f[s], p[(size_t)s * ps], acc);
    s_acc[grp][t % kMergeDims] = acc;
    __syncthreads();
    if (grp == 0) {
        float tot = s_acc[0][t];
        for (int i = 1; i < NG; ++i)
            tot += s_acc[i][t];
        a.out[(size_t)h * DH + d] = tot / L;
    }
}

template <int DH, int G>
hipError_t go(const AttendArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((k_attend<DH, G>), dim3(a.n_split, a.kv_heads), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (a.n_split > kMaxSplits)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_merge<DH, G>), dim3(a.kv_heads * G, DH / kMergeDims), dim3(kMergeThreads),
                       0, s, a);
    return hipGetLastError();
}

template <int DH>
hipError_t go_g(const AttendArgs &a, int G, hipStream_t s)
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

hipError_t launch_attend(const AttendArgs &a, int Dh, int G, hipStream_t s)
{
    switch (Dh) {
    case 64: return go_g<64>(a, G, s);
    case 128: return go_g<128>(a, G, s);
    case 256: return go_g<256>(a, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace qsa
