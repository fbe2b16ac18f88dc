// qsa_internal.h -- shared definitions of the gfx950 QSA kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kHistBits = 12;       // first radix digit of the top-k key
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCellsPerSplit = 64;  // cells handled by one attention workgroup

// Control words at the start of the workspace.
enum Ctrl : int { kCtrlSelectDone = 0, kCtrlCandCount = 1, kCtrlWords = 64 };

// Workspace carve-up.  ctrl and hist are contiguous so one fill clears both.
struct WsLayout {
    size_t ctrl, hist, bitmap, keys, cand, sel, part, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(int64_t max_blocks, int64_t sel_entries, int64_t part_floats)
{
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.ctrl = take(sizeof(uint32_t) * kCtrlWords);
    L.hist = take(sizeof(uint32_t) * kHistBins);
    L.bitmap = take(sizeof(uint64_t) * (size_t)((max_blocks + 63) / 64));
    L.keys = take(sizeof(uint32_t) * (size_t)max_blocks);
    L.cand = take(sizeof(uint64_t) * (size_t)max_blocks);
    L.sel = take(sizeof(int32_t) * (size_t)sel_entries);
    L.part = take(sizeof(float) * (size_t)part_floats);
    L.total = off;
    return L;
}

// Floats of one attention partial: m[G], l[G], acc[G][Dh].
__host__ __device__ inline int64_t part_stride(int G, int Dh) { return 2 * (int64_t)G + (int64_t)G * Dh; }

inline int64_t n_splits(int64_t n_cells) { return (n_cells + kCellsPerSplit - 1) / kCellsPerSplit; }

// ------------------------------------------------------------- launchers
struct UpdateArgs {
    void *idx_k;
    void *summary;
    uint16_t *k;
    uint16_t *v;
    const void *new_idx_row;    // appended raw indexer-key row (null: no append)
    const uint16_t *new_k_row;
    const uint16_t *new_v_row;
    const float *gamma;
    uint32_t *clear_ptr;        // zero [clear_ptr, clear_ptr + clear_words) (null: none)
    int32_t clear_words;
    int32_t idx_row_words;      // 32-bit words in one raw indexer-key row
    int32_t kv_row_words;       // 32-bit words in one K (or V) row
    int64_t pos;                // append position (ignored without new_idx_row)
    int32_t b0, nblk;           // pool blocks [b0, b0 + nblk)
    int32_t H, D;
    double eps, theta;
};
hipError_t launch_update(const UpdateArgs &a, bool f16, hipStream_t s);

struct ScoreArgs {
    const void *summary;
    const float *q;
    const float *w;
    float *scores;              // optional fp32 scores
    uint32_t *keys;             // optional order-preserving keys
    uint32_t *hist;             // optional histogram of the key's top 12 bits
    int32_t nb;
    int32_t D;
};
hipError_t launch_score(const ScoreArgs &a, bool f16, int row_bytes, hipStream_t s);

hipError_t launch_keys_hist(const float *scores, int32_t nb, uint32_t *keys, uint32_t *hist,
                            hipStream_t s);
hipError_t launch_fill_zero(uint32_t *p, int32_t words, hipStream_t s);
hipError_t launch_iota(int32_t *p, int32_t n, hipStream_t s);

struct SelectArgs {
    const uint32_t *keys;
    const uint32_t *hist;
    uint32_t *ctrl;
    uint64_t *bitmap;
    uint64_t *cand;
    int32_t *sel;
    int32_t nb;
    int32_t k;
};
hipError_t launch_select(const SelectArgs &a, hipStream_t s);

struct AttendArgs {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *sel;         // null: every block kept (cell e = e)
    const float *q;
    float *part;
    float *out;
    int32_t n_sel_blocks;
    int32_t nb;                 // floor(n_tokens / 4)
    int32_t n_cells;
    int32_t n_split;
    int32_t kv_heads;
    float scale;
};
hipError_t launch_attend(const AttendArgs &a, int Dh, int G, hipStream_t s);

}  // namespace qsa
