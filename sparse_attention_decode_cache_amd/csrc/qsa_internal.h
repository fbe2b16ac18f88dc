// qsa_internal.h -- shared definitions of the gfx950 QSA kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kListDiv = 8;         // per-tile top-k lists keep R / 8 entries or more (up to R / 2)

// Workspace carve-up.  The histogram region (decode step) is optional:
// hist_splits > 0 sizes its per-split id staging.
struct WsLayout {
    size_t keys, lists, sel, part;
    size_t ctrl, hist, bmax, bminc, last, stage, stage_n;   // 0 without the histogram region
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kHistBins = 2048, kHistLast = 64;   // qsa_hist.h

inline WsLayout ws_layout(int64_t max_blocks, int64_t sel_entries, int64_t part_floats,
                          int64_t hist_splits = 0, int64_t k_blocks = 0)
{
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    if (hist_splits > 0)
        L.ctrl = take(256);     // first: the region's control words sit at a fixed offset
    L.keys = take(sizeof(uint32_t) * (size_t)max_blocks);
    L.lists = take(sizeof(uint64_t) * (size_t)((max_blocks + 1) / 2 + 64));
    L.sel = take(sizeof(int32_t) * (size_t)sel_entries);
    L.part = take(sizeof(float) * (size_t)part_floats);
    if (hist_splits > 0) {
        L.hist = take(sizeof(uint32_t) * kHistBins);
        L.bmax = take(sizeof(uint64_t) * kHistBins);
        L.bminc = take(sizeof(uint64_t) * kHistBins);
        L.last = take(sizeof(uint64_t) * kHistLast);
        L.stage = take(sizeof(int32_t) * (size_t)(hist_splits * k_blocks));
        L.stage_n = take(sizeof(int32_t) * (size_t)hist_splits);
    }
    L.total = off;
    return L;
}

// Floats of one attention partial: m[G], l[G], acc[G][Dh].
__host__ __device__ inline int64_t part_stride(int G, int Dh) { return 2 * (int64_t)G + (int64_t)G * Dh; }
// The decode-step kernel's partial: acc[G][Dh], m[G], l[G], padded to 16 bytes.
__host__ __device__ inline int64_t dec_part_stride(int G, int Dh)
{
    return ((int64_t)G * Dh + 2 * (int64_t)G + 3) / 4 * 4;
}

// Cells handled by one attention workgroup.
constexpr int kCellsPerSplit = 16;

inline int64_t n_splits(int64_t n_cells)
{
    return (n_cells + kCellsPerSplit - 1) / kCellsPerSplit;
}

// Cells per iteration of the attention unit of the chunk / batch / masked
// kernels (qsa_unit.h).
constexpr int kUnitCells = 64;

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
    int32_t n_new;              // rows appended at pos .. pos + n_new - 1 (with new_idx_row)
    int32_t b0, nblk;           // pool blocks [b0, b0 + nblk)
    int32_t H, D;
    double eps, theta;
};
hipError_t launch_update(const UpdateArgs &a, bool f16, hipStream_t s);

// Histogram insertion by the score pass (see qsa_hist.h); off when hist is null.
struct HistOut {
    uint32_t *hist;             // [hist::kBins] counts (cleared by the previous call)
    uint64_t *bmax;             // [hist::kBins] largest composite per bin
    uint64_t *bminc;            // [hist::kBins] complement of the smallest composite per bin
    uint64_t *last;             // [hist::kLast] maxima of the tiles' last list entries
    void *ctrl;                 // hist::Ctrl: window feedback in, tag / sigma / window out
    const float *gamma;         // [D] RMSNorm weights (for sigma)
    uint64_t epoch;             // this call's epoch (the tag stamp)
    float def_k, def_top;       // kappa / sigma and top / sigma when no feedback is usable
};

struct ScoreArgs {
    const void *summary;
    const float *q;
    const float *w;
    float *scores;              // optional fp32 scores
    uint32_t *keys;             // optional order-preserving keys
    uint64_t *lists;            // optional per-tile top-T composites (with keys)
    int32_t list_t;             // T: entries per tile list (with lists)
    int32_t nb;
    int32_t D;
    int32_t fuse;               // workgroup 0 first runs `upd` (append, pool <= 1 row)
    UpdateArgs upd;
    HistOut h;                  // histogram insertion (lists required)
};
hipError_t launch_score(const ScoreArgs &a, bool f16, int row_bytes, hipStream_t s);

// Batched calls: per-sequence arguments travel in the kernel arguments.
constexpr int kMaxBatch = 8;
struct ScoreBatchArgs {
    int32_t n;
    int32_t tile0[kMaxBatch + 1];   // first workgroup of each sequence (filled by the launcher)
    ScoreArgs seq[kMaxBatch];
};
hipError_t launch_score_batch(ScoreBatchArgs &b, bool f16, int row_bytes, hipStream_t s);
// Rows per score workgroup (tile) for a given indexer row size.
int score_tile_rows(bool f16, int row_bytes);

// Several queries of one sequence (consecutive tokens: speculative verify)
// scored in one pass over the summary rows.  Query i sees blocks [0, nbq[i]);
// every summary row is loaded once and dotted with every query.
constexpr int kMaxMulti = 4;
struct ScoreMultiArgs {
    const void *summary;
    int32_t nb;                     // rows streamed: the last query's blocks
    int32_t D;
    int32_t fuse;                   // workgroup 0 first runs `upd` (append, pool <= 1 row)
    UpdateArgs upd;
    int32_t nbq[kMaxMulti];         // blocks seen by query i (<= nb)
    const float *q[kMaxMulti];      // [H][D] fp32 per query
    const float *w[kMaxMulti];      // [H] per query
    uint32_t *keys[kMaxMulti];      // optional per query: [nb] order-preserving keys
    uint64_t *lists[kMaxMulti];     // optional per query: per-tile top-T composites
    float *scores;                  // optional [n_q][ld_scores]: -inf at b >= nbq[i]
    int64_t ld_scores;
    int32_t list_t;                 // T: entries per tile list (with lists)
    HistOut h;                      // one query only: histogram insertion of its lists
};
hipError_t launch_score_multi(const ScoreMultiArgs &a, int n_q, bool f16, int row_bytes,
                              hipStream_t s);

// Keys and per-tile lists (R = 256) from given fp32 scores.
constexpr int kKeysTile = 256;
hipError_t launch_keys(const float *scores, int32_t nb, uint32_t *keys, uint64_t *lists,
                       hipStream_t s);
hipError_t launch_fill_zero(uint32_t *p, int32_t words, hipStream_t s);
// The former cell-level path: block scores expanded to cells; tail cells appended.
hipError_t launch_expand_cells(const float *scores, int32_t nb, float *cells, hipStream_t s);
hipError_t launch_tail_cells(int32_t *cells, int32_t at, int32_t nb, int32_t tail, hipStream_t s);
hipError_t launch_iota(int32_t *p, int32_t n, hipStream_t s);

// Per-tile candidate lists: a tile of R consecutive blocks keeps its T = R/8
// largest composite keys, sorted descending, zero-filled past the tile's
// blocks (a composite is never 0).  R depends on the producer.
struct SelectArgs {
    const uint32_t *keys;       // [nb] order-preserving score keys (16-byte aligned)
    const uint64_t *lists;      // [ntiles * T] composites, descending per tile
    int32_t *sel;
    int32_t nb;
    int32_t k;
    int32_t ntiles;
    int32_t T;
    int32_t lkeys_off;          // byte offset of an nb-word key cache in the dynamic LDS (0: none;
                                // set by the launchers when it fits)
    int32_t pad_to;             // batch select, nb <= k: slots [nb, pad_to) of sel get -1
};
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
struct SelectBatchArgs {
    int32_t n;
    SelectArgs seq[kMaxBatch];
};
hipError_t launch_select_batch(const SelectBatchArgs &b, hipStream_t s);

// Order-preserving 32-bit key of an fp32 score: larger scores give larger
// keys; -0 and +0 must compare equal, so -0 is folded into +0 first.
__device__ inline uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score an order-preserving key was made from (-0 was folded into +0).
__device__ inline float key_score(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__host__ __device__ inline uint64_t comp_key(uint32_t key, uint32_t id)
{
    return ((uint64_t)key << 32) | (uint64_t)(~id);
}

struct AttendArgs {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *sel;         // null: every block kept (cell e = e)
    const float *q;
    float *part;
    float *out;
    int32_t n_sel_blocks;
    int32_t nb;                 // floor(n_tokens / 4)
    int32_t n_cells;            // cells of the attention splits
    int32_t n_tail;             // cells 4*nb + j, j < n_tail, folded in by the merge
    int32_t n_split;            // splits per KV head (partials [kv_heads][n_split])
    int32_t kv_heads;
    float scale;
};
hipError_t launch_attend(const AttendArgs &a, int Dh, int G, hipStream_t s);
// The same over a q8_0 K/V cache: a.k / a.v hold the int8 codes
// ([rows][kv_heads][Dh]), the scales are [rows][kv_heads][Dh/32] binary16;
// the merge reads the a.n_tail tail rows (if any) in the same format.
hipError_t launch_attend_q8(const AttendArgs &a, const uint16_t *k_scales, const uint16_t *v_scales,
                            int Dh, int G, hipStream_t s);
// q8_0 quantisation of n_blocks blocks of 32 binary16 values.
hipError_t launch_q8_0_quantize(const uint16_t *x, int64_t n_blocks, int8_t *codes, uint16_t *scales,
                                hipStream_t s);
struct AttendBatchArgs {
    int32_t n;
    int32_t wg0[kMaxBatch + 1];     // first workgroup of each sequence (filled by the launcher)
    AttendArgs seq[kMaxBatch];
};
// The batch's attention: each sequence's cells in 64-cell iterations, one
// per workgroup, then a merge of the partials (n_split is set here).
hipError_t launch_attend_batch(AttendBatchArgs &b, int Dh, int G, hipStream_t s);
// The merge of a batch's split partials (one load round per output slice).
hipError_t launch_merge_batch(const AttendBatchArgs &b, int Dh, int G, hipStream_t s);
// The same merge for a prefill chunk of n_q queries split n_split ways each.
hipError_t launch_merge_chunk(float *part, float *out, int n_q, int kv_heads, int n_split, int Dh,
                              int G, hipStream_t s);
// Stages 3 + 4 fused: every attention workgroup selects (a.sel is ignored;
// the chosen ids come from `sa`, sa.sel optionally receives them all).
hipError_t launch_select_attend(const AttendArgs &a, const SelectArgs &sa, int Dh, int G,
                                hipStream_t s);

// Stages 3 + 4 of the decode step in one kernel after a score pass with
// histogram insertion: grid (ns splits, kv_heads), 1024 threads.  Split s
// owns the tiles [s ntiles / ns, (s + 1) ntiles / ns); it finds kappa from
// the histogram, attends the cells of its own winners, publishes its partial
// and a flag; the first workgroups of each KV head merge, one workgroup
// clears the histogram for the next call.  Falls back to the full top-k of
// qsa_select.h (every workgroup, slots dealt out evenly) when the histogram
// cannot decide.
constexpr int kDecodeThreads = 1024;
constexpr int kDecodeMaxSplits = 128;
struct DecodeArgs {
    const uint16_t *k;
    const uint16_t *v;
    const float *q;
    float *out;
    int32_t *sel_out;           // optional: all chosen ids, ascending
    int32_t nb, n_tail, kv_heads, k_blocks;
    float scale;
    SelectArgs sa;              // keys and tile lists of the score pass (sa.sel unused)
    const uint32_t *hist;
    const uint64_t *bmax;
    const uint64_t *bminc;
    const uint64_t *last;
    void *ctrl;                 // hist::Ctrl
    int32_t ns;                 // splits per KV head
    float *part;                // [kv_heads][ns] partials
    int32_t *stage;             // [ns][k_blocks] each split's winners, ascending (sel_out only)
    int32_t *stage_n;           // [ns]
    uint64_t epoch;             // unique per call
};
// The attention kernel (grid ns x kv_heads) and then the merge kernel.
hipError_t launch_decode_attend(const DecodeArgs &a, int Dh, int G, hipStream_t s);
// Whether that kernel takes nb blocks at these shapes (its LDS, the full
// top-k's overlay included, fits a workgroup).
bool decode_fits(int64_t nb, int Dh, int G);

// ------------------------------------------------------------ prefill chunk
// n_q consecutive tokens of one sequence in one call: query i sits at position
// n0 + i and sees the blocks completed by then.
constexpr int kChunkWgTarget = 512;     // attention workgroups aimed at when queries are few
constexpr int kChunkMaxSplits = 64;
constexpr int kChunkMaxIds = 4096;      // block ids of one query (k <= 4095)

struct ChunkArgs {
    void *idx_k;                // cache: raw indexer keys, summaries, K, V
    const void *summary;
    uint16_t *k;
    uint16_t *v;
    const void *idx_rows;       // [n_q] appended rows
    const uint16_t *k_rows;
    const uint16_t *v_rows;
    int32_t idx_row_bytes;
    int32_t kv_row_bytes;
    const float *q_idx;         // [n_q][H][D]
    const float *w;             // [n_q][H]
    const float *q;             // [n_q][Hq][Dh]
    float *out;                 // [n_q][Hq][Dh]
    int32_t *sel_out;           // optional [n_q][kb]
    float *scores_out;          // optional [n_q][nb_last]
    _Float16 *qhl;              // workspace: folded queries, MFMA operand layout, padded with
                                // zeros to whole groups of 128 queries
    float *qscale;              // workspace: [n_q] power-of-two factors
    uint32_t *keys;             // workspace: [n_q][ldk]
    int32_t *sel;               // workspace: [n_q][kb]
    float *part;                // workspace: attention partials (n_split > 1)
    int64_t ldk;
    int32_t n0, n_q, nb_last, kb;   // kb: blocks kept per query
    int32_t H, D;
    int32_t kv_heads, n_split;
    float scale;
    // grouped-union attention (k_union.hip) instead of the per-query one when
    // union_q > 0: groups of union_q consecutive queries
    int32_t union_q;
    int32_t ucap;               // union entries per group (>= union_q * kb)
    int32_t *uni;               // workspace: [groups][ucap] union block ids, ascending
    uint32_t *umask;            // workspace: [groups][ucap] queries (bits) that chose each
    int32_t *ucount;            // workspace: [groups] union sizes
};
// Grouped-union attention of a chunk: the union build, then the attention.
constexpr size_t kUnionBuildLds = 128 * 1024;
constexpr int kUnionMaxQ = 32;          // queries of a group (bits of a union block's mask)
constexpr int kUnionMaxRows = 64;       // query x head rows of a group (four matrix-core tiles)
size_t union_build_lds(int qg, int32_t nb_last);
hipError_t launch_union(const ChunkArgs &c, int Dh, int G, hipStream_t s);
// The gather switched off (an ablation of the selected K/V gather): flash-
// decode over every cached K / V row, the blocks outside `sel` masked out of
// the softmax.  Same cells as the gathered attention.
constexpr int kMaskedSplits = 256;      // per KV head: 512 workgroups for two KV heads
constexpr int kMaskedMaxSplits = 1024;
struct MaskedArgs {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *sel;         // [n_sel_blocks] ascending
    const float *q;
    float *out;
    float *part;                // [kv_heads][n_split] partials
    uint32_t *bitmap;           // [ceil(nb / 32)] words, written by the launch
    int64_t n_tokens;
    int32_t n_sel_blocks;
    int32_t kv_heads;
    int32_t n_split;            // set by the launcher
    float scale;
};
hipError_t launch_masked_attend(MaskedArgs m, int Dh, int G, hipStream_t s);

// Append, then (after the caller's pooling launch) score, select and attend.
hipError_t launch_chunk_append(const ChunkArgs &c, hipStream_t s);
hipError_t launch_chunk_rest(ChunkArgs c, bool f16, int Dh, int G, hipStream_t s);

}  // namespace qsa
