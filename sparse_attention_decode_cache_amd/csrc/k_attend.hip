// k_attend.hip -- stage 4: attention over the gathered cells only.
//
// [post 10, "selected QSA K/V gather（COMMON-005）"]: only the K/V rows of the
// chosen cells (4 per chosen block, plus the tail of the unfinished block) are
// read, and ordinary softmax attention runs over them.  The gather is not
// materialised: the attention workgroups load the selected rows directly.
//
// Split-context flash decode.  Cells are enumerated e = 0..n_cells-1 (chosen
// blocks ascending, 4 cells each, then the tail when the splits hold it).
// Workgroup (split, g) takes 16 consecutive cells of KV head g for all G
// query heads of the group (GQA: each K/V row is read once for G heads) with
// the tile routine of qsa_attend.h: 2048 chosen cells and 2 KV heads make 256
// workgroups, one per CU, and the merge folds in the <= 3 tail cells.  The
// split's partial (m, l, acc) goes to the workspace; a second kernel merges
// the partials of a head (one global latency round, fixed order: bitwise
// repeatable).
#include "qsa_attend.h"
#include "qsa_internal.h"
#include "qsa_merge.h"
#include "qsa_select.h"
#include "qsa_wave.h"

namespace qsa {
namespace {

using namespace att;
using namespace mrg;

// Split `split` of KV head g with the partial written to the workspace.
template <int DH, int G, bool Q8 = false>
__device__ void attend_split(const AttendArgs &a, AttLds<DH, G> &L, int split, int g, Q8Scales q8 = {})
{
    attend_tile<DH, G, Q8>(a, L, L.blk, split * kCells, g, [&](AttLds<DH, G> &T) {
        float *part = a.part + ((size_t)g * a.n_split + split) * (size_t)part_stride(G, DH);
        for (int i = threadIdx.x; i < G * DH; i += kAT)
            part[2 * G + i] = tile_acc<DH, G>(T, i);
        if (threadIdx.x < G) {
            part[threadIdx.x] = T.m[threadIdx.x];
            part[G + threadIdx.x] = T.l[threadIdx.x];
        }
    }, q8);
}

template <int DH, int G>
__global__ __launch_bounds__(kAT) void k_attend(AttendArgs a)
{
    __shared__ AttLds<DH, G> L;
    const int split = blockIdx.x;
    // the split's block ids (identity when every block is kept)
    if (threadIdx.x < kCells / 4) {
        const int i = split * (kCells / 4) + threadIdx.x;
        L.blk[threadIdx.x] = !a.sel ? i : (i < a.n_sel_blocks ? a.sel[i] : -1);
    }
    __syncthreads();
    attend_split<DH, G>(a, L, split, blockIdx.y);
}

// The same splits over a q8_0 K/V cache (codes in a.k / a.v, scales in q8).
template <int DH, int G>
__global__ __launch_bounds__(kAT) void k_attend_q8(AttendArgs a, Q8Scales q8)
{
    __shared__ AttLds<DH, G> L;
    const int split = blockIdx.x;
    if (threadIdx.x < kCells / 4) {
        const int i = split * (kCells / 4) + threadIdx.x;
        L.blk[threadIdx.x] = !a.sel ? i : (i < a.n_sel_blocks ? a.sel[i] : -1);
    }
    __syncthreads();
    attend_split<DH, G, true>(a, L, split, blockIdx.y, q8);
}

// Stages 3 and 4 in one kernel: every attention workgroup runs the top-k
// routine itself (the same deterministic result everywhere, each on its own
// CU in parallel) and keeps the ids of its own 4 slots; workgroup (0, 0) also
// writes the whole list when the caller asked for it.  No select launch and
// no round trip of the id list through memory.
struct FusedArgs {
    AttendArgs att;
    SelectArgs sel;             // sel.sel: optional output of all k ids
};

template <int DH, int G>
__global__ __launch_bounds__(kAT) void k_select_attend(FusedArgs f)
{
    static_assert(kAT == sel::kT, "one workgroup size for both stages");
    __shared__ AttLds<DH, G> L;
    extern __shared__ uint4 sel_lds[];
    const int split = blockIdx.x;
    if (threadIdx.x < kCells / 4)
        L.blk[threadIdx.x] = -1;
    __syncthreads();
    const uint32_t s0 = (uint32_t)split * (kCells / 4);
    int32_t *all = (blockIdx.x == 0 && blockIdx.y == 0) ? f.sel.sel : nullptr;
    int32_t *blk = L.blk;
    sel::run(f.sel, reinterpret_cast<char *>(sel_lds), [=](uint32_t slot, uint32_t id) {
        if (slot - s0 < (uint32_t)(kCells / 4))
            blk[slot - s0] = (int32_t)id;
        if (all)
            all[slot] = (int32_t)id;
    });
    __syncthreads();
    attend_split<DH, G>(f.att, L, split, blockIdx.y);
}

template <int DH, int G>
__global__ __launch_bounds__(kMT) void k_merge(AttendArgs a)
{
    __shared__ MergeLds ml;
    merge_unit<DH, G>(a, ml, blockIdx.x, blockIdx.y);
}

template <int DH, int G>
__global__ __launch_bounds__(kMT) void k_merge_q8(AttendArgs a, Q8Scales q8)
{
    __shared__ MergeLds ml;
    merge_unit<DH, G, true>(a, ml, blockIdx.x, blockIdx.y, q8);
}

// A batch: grid (sequence x query head, 64-dim slice), over each sequence's
// split partials.
template <int DH, int G>
__global__ __launch_bounds__(kMT) void k_merge_batch(AttendBatchArgs b)
{
    __shared__ MergeLds ml;
    const int hq = b.seq[0].kv_heads * G;
    const int s = (int)blockIdx.x / hq;
    merge_unit<DH, G>(b.seq[s], ml, (int)blockIdx.x % hq, blockIdx.y);
}

// Prefill chunk with few queries: grid (query x query head, 64-dim slice);
// query i's partials are [kv_heads][n_split] at part + i * kv_heads * n_split
// partials, its output [Hq][DH] at out + i * Hq * DH.
struct ChunkMergeArgs {
    float *part;
    float *out;
    int32_t kv_heads, n_split;
};

template <int DH, int G>
__global__ __launch_bounds__(kMT) void k_merge_chunk(ChunkMergeArgs m)
{
    __shared__ MergeLds ml;
    const int hq = m.kv_heads * G;
    const int i = (int)blockIdx.x / hq;
    AttendArgs a{};
    a.part = m.part + (size_t)i * m.kv_heads * m.n_split * part_stride(G, DH);
    a.out = m.out + (size_t)i * hq * DH;
    a.n_split = m.n_split;
    a.kv_heads = m.kv_heads;
    merge_unit<DH, G>(a, ml, (int)blockIdx.x % hq, blockIdx.y);
}

template <int DH, int G>
hipError_t merge(const AttendArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((k_merge<DH, G>), dim3(a.kv_heads * G, DH / kWave), dim3(kMT), 0, s, a);
    return hipGetLastError();
}

template <int DH, int G>
hipError_t merge_q8(const AttendArgs &a, const Q8Scales &q8, hipStream_t s)
{
    hipLaunchKernelGGL((k_merge_q8<DH, G>), dim3(a.kv_heads * G, DH / kWave), dim3(kMT), 0, s, a,
                       q8);
    return hipGetLastError();
}

template <int DH, int G>
hipError_t go(const AttendArgs &a, const SelectArgs *sa, hipStream_t s)
{
    if (a.n_split > kMaxSplits)
        return hipErrorInvalidValue;
    if (!sa) {
        hipLaunchKernelGGL((k_attend<DH, G>), dim3(a.n_split, a.kv_heads), dim3(kAT), 0, s, a);
    } else {
        SelectArgs sc = *sa;
        const size_t lds = sel::lds_with_cache(sc, sc.nb, sel::kMaxLds - sizeof(AttLds<DH, G>));
        if (lds + sizeof(AttLds<DH, G>) > sel::kMaxLds)
            return hipErrorInvalidValue;
        if (lds > 32 * 1024) {
            static hipError_t attr = hipFuncSetAttribute(
                (const void *)k_select_attend<DH, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                (int)(sel::kMaxLds - sizeof(AttLds<DH, G>)));
            if (attr != hipSuccess)
                return attr;
        }
        FusedArgs f{a, sc};
        hipLaunchKernelGGL((k_select_attend<DH, G>), dim3(a.n_split, a.kv_heads), dim3(kAT), lds, s,
                           f);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return merge<DH, G>(a, s);
}

template <int DH>
hipError_t go_g(const AttendArgs &a, const SelectArgs *sa, int G, hipStream_t s)
{
    switch (G) {
    case 1: return go<DH, 1>(a, sa, s);
    case 2: return go<DH, 2>(a, sa, s);
    case 4: return go<DH, 4>(a, sa, s);
    case 8: return go<DH, 8>(a, sa, s);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch(const AttendArgs &a, const SelectArgs *sa, int Dh, int G, hipStream_t s)
{
    switch (Dh) {
    case 64: return go_g<64>(a, sa, G, s);
    case 128: return go_g<128>(a, sa, G, s);
    case 256: return go_g<256>(a, sa, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend(const AttendArgs &a, int Dh, int G, hipStream_t s)
{
    return dispatch(a, nullptr, Dh, G, s);
}

hipError_t launch_merge_chunk(float *part, float *out, int n_q, int kv_heads, int n_split, int Dh,
                              int G, hipStream_t s)
{
    if (n_q < 1 || n_split < 1 || n_split > kMaxSplits)
        return hipErrorInvalidValue;
    const ChunkMergeArgs m{part, out, kv_heads, n_split};
    const dim3 grid((unsigned)(n_q * kv_heads * G), (unsigned)(Dh / kWave));
#define QSA_MERGE_G(DHV)                                                                \
    switch (G) {                                                                        \
    case 1: hipLaunchKernelGGL((k_merge_chunk<DHV, 1>), grid, dim3(kMT), 0, s, m); break; \
    case 2: hipLaunchKernelGGL((k_merge_chunk<DHV, 2>), grid, dim3(kMT), 0, s, m); break; \
    case 4: hipLaunchKernelGGL((k_merge_chunk<DHV, 4>), grid, dim3(kMT), 0, s, m); break; \
    case 8: hipLaunchKernelGGL((k_merge_chunk<DHV, 8>), grid, dim3(kMT), 0, s, m); break; \
    default: return hipErrorInvalidValue;                                               \
    }                                                                                   \
    break;
    switch (Dh) {
    case 64: QSA_MERGE_G(64)
    case 128: QSA_MERGE_G(128)
    case 256: QSA_MERGE_G(256)
    default: return hipErrorInvalidValue;
    }
#undef QSA_MERGE_G
    return hipGetLastError();
}

hipError_t launch_merge_batch(const AttendBatchArgs &b, int Dh, int G, hipStream_t s)
{
    if (b.n < 1 || b.n > kMaxBatch)
        return hipErrorInvalidValue;
    for (int i = 0; i < b.n; ++i)
        if (b.seq[i].n_split < 1 || b.seq[i].n_split > kMaxSplits || b.seq[i].kv_heads != b.seq[0].kv_heads)
            return hipErrorInvalidValue;
    const dim3 grid((unsigned)(b.n * b.seq[0].kv_heads * G), (unsigned)(Dh / kWave));
#define QSA_MERGE_G(DHV)                                                                \
    switch (G) {                                                                        \
    case 1: hipLaunchKernelGGL((k_merge_batch<DHV, 1>), grid, dim3(kMT), 0, s, b); break; \
    case 2: hipLaunchKernelGGL((k_merge_batch<DHV, 2>), grid, dim3(kMT), 0, s, b); break; \
    case 4: hipLaunchKernelGGL((k_merge_batch<DHV, 4>), grid, dim3(kMT), 0, s, b); break; \
    case 8: hipLaunchKernelGGL((k_merge_batch<DHV, 8>), grid, dim3(kMT), 0, s, b); break; \
    default: return hipErrorInvalidValue;                                               \
    }                                                                                   \
    break;
    switch (Dh) {
    case 64: QSA_MERGE_G(64)
    case 128: QSA_MERGE_G(128)
    case 256: QSA_MERGE_G(256)
    default: return hipErrorInvalidValue;
    }
#undef QSA_MERGE_G
    return hipGetLastError();
}

hipError_t launch_attend_q8(const AttendArgs &a, const uint16_t *k_scales, const uint16_t *v_scales,
                            int Dh, int G, hipStream_t s)
{
    if (a.n_tail < 0 || a.n_tail > 3 || a.n_split < 1 || a.n_split > kMaxSplits)
        return hipErrorInvalidValue;
    const Q8Scales q8{k_scales, v_scales};
    const dim3 grid((unsigned)a.n_split, (unsigned)a.kv_heads);
#define QSA_Q8_G(DHV)                                                                             \
    switch (G) {                                                                                  \
    case 1: hipLaunchKernelGGL((k_attend_q8<DHV, 1>), grid, dim3(kAT), 0, s, a, q8); break;       \
    case 2: hipLaunchKernelGGL((k_attend_q8<DHV, 2>), grid, dim3(kAT), 0, s, a, q8); break;       \
    case 4: hipLaunchKernelGGL((k_attend_q8<DHV, 4>), grid, dim3(kAT), 0, s, a, q8); break;       \
    case 8: hipLaunchKernelGGL((k_attend_q8<DHV, 8>), grid, dim3(kAT), 0, s, a, q8); break;       \
    default: return hipErrorInvalidValue;                                                         \
    }                                                                                             \
    break;
    switch (Dh) {
    case 64: QSA_Q8_G(64)
    case 128: QSA_Q8_G(128)
    case 256: QSA_Q8_G(256)
    default: return hipErrorInvalidValue;
    }
#undef QSA_Q8_G
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (Dh * 16 + G) {
    case 64 * 16 + 1: return merge_q8<64, 1>(a, q8, s);
    case 64 * 16 + 2: return merge_q8<64, 2>(a, q8, s);
    case 64 * 16 + 4: return merge_q8<64, 4>(a, q8, s);
    case 64 * 16 + 8: return merge_q8<64, 8>(a, q8, s);
    case 128 * 16 + 1: return merge_q8<128, 1>(a, q8, s);
    case 128 * 16 + 2: return merge_q8<128, 2>(a, q8, s);
    case 128 * 16 + 4: return merge_q8<128, 4>(a, q8, s);
    case 128 * 16 + 8: return merge_q8<128, 8>(a, q8, s);
    case 256 * 16 + 1: return merge_q8<256, 1>(a, q8, s);
    case 256 * 16 + 2: return merge_q8<256, 2>(a, q8, s);
    case 256 * 16 + 4: return merge_q8<256, 4>(a, q8, s);
    case 256 * 16 + 8: return merge_q8<256, 8>(a, q8, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_select_attend(const AttendArgs &a, const SelectArgs &sa, int Dh, int G,
                                hipStream_t s)
{
    if (sa.T != 8 && sa.T != 16 && sa.T != 32)
        return hipErrorInvalidValue;
    return dispatch(a, &sa, Dh, G, s);
}

}  // namespace qsa
