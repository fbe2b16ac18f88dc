// qsa_api.hip -- the C ABI declared in include/qsa.h: argument checks,
// workspace carve-up and the launch sequence of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "qsa_internal.h"
#include "qsa_select.h"

using namespace qsa;

namespace {

thread_local char tl_err[512] = "";

qsa_status fail(qsa_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(tl_err, sizeof(tl_err), fmt, ap);
    va_end(ap);
    return s;
}

qsa_status ok()
{
    tl_err[0] = '\0';
    return QSA_OK;
}

qsa_status hip_fail(hipError_t e, const char *where)
{
    return fail(QSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(int32_t dtype) { return dtype == QSA_F16 ? 2 : 4; }

qsa_status check_desc(const qsa_layer_desc *d)
{
    if (!d)
        return fail(QSA_ERR_ARG, "desc is NULL");
    if (d->block != 4)
        return fail(QSA_ERR_UNSUPPORTED, "block must be 4 (got %d)", d->block);
    if (d->idx_dtype != QSA_F16 && d->idx_dtype != QSA_F32)
        return fail(QSA_ERR_UNSUPPORTED, "idx_dtype %d", d->idx_dtype);
    if (d->idx_heads != 1 && d->idx_heads != 4)
        return fail(QSA_ERR_UNSUPPORTED, "idx_heads must be 1 or 4 (got %d)", d->idx_heads);
    if (d->idx_dim != 64 && d->idx_dim != 128)
        return fail(QSA_ERR_UNSUPPORTED, "idx_dim must be 64 or 128 (got %d)", d->idx_dim);
    if (d->idx_heads * d->idx_dim * elem_bytes(d->idx_dtype) > 1024)
        return fail(QSA_ERR_UNSUPPORTED, "indexer row larger than 1024 bytes");
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
        return fail(QSA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", d->head_dim);
    if (d->kv_heads < 1 || d->q_heads < 1 || d->q_heads % d->kv_heads != 0)
        return fail(QSA_ERR_UNSUPPORTED, "q_heads %d not a multiple of kv_heads %d", d->q_heads,
                    d->kv_heads);
    const int G = d->q_heads / d->kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(QSA_ERR_UNSUPPORTED, "q_heads / kv_heads must be 1, 2, 4 or 8 (got %d)", G);
    if (d->top_k_tokens < 4 || d->top_k_tokens % 4 != 0 || d->top_k_tokens > 16380)
        return fail(QSA_ERR_UNSUPPORTED,
                    "top_k_tokens must be a positive multiple of 4, at most 16380 (got %d)",
                    d->top_k_tokens);
    if (!(d->rms_eps >= 0.0f) || !(d->rope_theta > 0.0f) || !(d->attn_scale >= 0.0f) ||
        !isfinite(d->rope_theta) || !isfinite(d->attn_scale))
        return fail(QSA_ERR_ARG, "rms_eps / rope_theta / attn_scale out of range");
    return QSA_OK;
}

qsa_status check_cache(const qsa_layer_cache *c, bool need_idx, bool need_sum, bool need_kv)
{
    if (!c)
        return fail(QSA_ERR_ARG, "cache is NULL");
    if (c->capacity < 4 || c->capacity % 4 != 0 || c->capacity > (1 << 21))
        return fail(QSA_ERR_ARG, "capacity must be a positive multiple of 4, <= 2^21 (got %d)",
                    c->capacity);
    if ((need_idx && (!c->idx_k || !aligned(c->idx_k, 16))) ||
        (need_sum && (!c->summary || !aligned(c->summary, 16))) ||
        (need_kv && (!c->k || !c->v || !aligned(c->k, 16) || !aligned(c->v, 16))))
        return fail(QSA_ERR_ARG, "cache pointer NULL or not 16-byte aligned");
    return QSA_OK;
}

float attn_scale(const qsa_layer_desc *d)
{
    return d->attn_scale > 0.0f ? d->attn_scale : 1.0f / sqrtf((float)d->head_dim);
}

int64_t decode_part_floats(const qsa_layer_desc *d)
{
    const int G = d->q_heads / d->kv_heads;
    const int64_t max_cells = (int64_t)d->top_k_tokens + 3;
    const int64_t a = n_splits(max_cells) * part_stride(G, d->head_dim);
    const int64_t b = (int64_t)kDecodeMaxSplits * dec_part_stride(G, d->head_dim);
    return (int64_t)d->kv_heads * (a > b ? a : b);
}

WsLayout decode_layout(const qsa_layer_desc *d, int32_t capacity)
{
    return ws_layout(capacity / 4, d->top_k_tokens / 4, decode_part_floats(d), kDecodeMaxSplits,
                     d->top_k_tokens / 4);
}

// Where the histogram window expects kappa, in units of the score scale, when
// no earlier call fed one back: where the k-th largest of nb normally
// distributed scores falls (the upper quantile k / nb, by bisection on the
// normal tail).  Any value is exact; a window that misses only costs that
// call the full top-k.
float default_kappa(int64_t nb, int64_t k)
{
    const double p = (double)k / (double)nb;        // < 1: there is a selection
    double lo = -10.0, hi = 10.0;
    for (int i = 0; i < 60; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (0.5 * erfc(mid / sqrt(2.0)) > p)
            lo = mid;
        else
            hi = mid;
    }
    return (float)(0.5 * (lo + hi));
}

// A distinct 56-bit value per decode-step call in this process (never 0):
// the score pass stamps the histogram region's tag with it and the attention
// kernel trusts the region only under its own call's stamp, so a tag left in
// a workspace by any earlier call never matches.
uint64_t next_epoch()
{
    static std::atomic<uint64_t> ctr{0};
    static const uint64_t base = [] {
        uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= (uint64_t)(uintptr_t)&ctr;
        x ^= x >> 33;
        x *= 0xff51afd7ed558ccdull;
        x ^= x >> 33;
        return x;
    }();
    uint64_t e;
    do {
        e = (base + ctr.fetch_add(1, std::memory_order_relaxed)) & ((1ull << 56) - 1);
    } while (e == 0);
    return e;
}

// Prefill-chunk workspace: folded queries, their scales, the keys of every
// (query, block), the chosen ids and the attention partials.
struct ChunkLayout {
    size_t qhl, qscale, keys, sel, part, uni, umask, ucount, total;
};

ChunkLayout chunk_layout(const qsa_layer_desc *d, int32_t capacity, int32_t n_q)
{
    ChunkLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t qk = (size_t)d->idx_heads * d->idx_dim;
    const size_t qpad = ((size_t)n_q + 127) / 128 * 128;   // whole groups of 128 queries
    const size_t ldk = ((size_t)capacity / 4 + 3) / 4 * 4;
    const int G = d->q_heads / d->kv_heads;
    L.qhl = take(qpad * qk * 2 * sizeof(uint16_t));
    L.qscale = take(sizeof(float) * (size_t)n_q);
    L.keys = take(sizeof(uint32_t) * (size_t)n_q * ldk);
    L.sel = take(sizeof(int32_t) * (size_t)n_q * (d->top_k_tokens / 4));
    L.part = take(sizeof(float) * 2 * (size_t)kChunkWgTarget * part_stride(G, d->head_dim));
    // the grouped-union lists: ceil(n_q / qg) groups of qg <= kUnionMaxQ
    // queries' ids each
    const size_t uents = ((size_t)n_q + kUnionMaxQ) * (size_t)(d->top_k_tokens / 4);
    L.uni = take(sizeof(int32_t) * uents);
    L.umask = take(sizeof(uint32_t) * uents);
    L.ucount = take(sizeof(int32_t) * (size_t)n_q);
    L.total = off;
    return L;
}

// Queries per group of the grouped-union attention: as many as fill 64
// query x head rows (four matrix-core tiles), at most 32 (the bits of a
// union block's mask), fewer when their bitmaps would not fit the union
// build's LDS.
int union_group(const qsa_layer_desc *d, int32_t nb_last)
{
    const int G = d->q_heads / d->kv_heads;
    int qg = kUnionMaxRows / G < kUnionMaxQ ? kUnionMaxRows / G : kUnionMaxQ;
    while (qg > 1 && union_build_lds(qg, nb_last) > kUnionBuildLds)
        --qg;
    return qg >= 1 && union_build_lds(qg, nb_last) <= kUnionBuildLds ? qg : 0;
}

qsa_status check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (!ws || !aligned(ws, 256))
        return fail(QSA_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
    if (ws_bytes < need)
        return fail(QSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return QSA_OK;
}

// Compute units of the current device (cached per device).
int64_t device_cus()
{
    static thread_local int cached_dev = -1;
    static thread_local int64_t cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

AttendArgs attend_args(const qsa_layer_desc *d, const qsa_layer_cache *c, int32_t n_tokens,
                       const int32_t *sel, int32_t n_sel_blocks, const float *q, float *out,
                       float *part)
{
    AttendArgs a{};
    a.k = c->k;
    a.v = c->v;
    a.sel = sel;
    a.q = q;
    a.part = part;
    a.out = out;
    a.n_sel_blocks = n_sel_blocks;
    a.nb = n_tokens / 4;
    a.n_cells = 4 * n_sel_blocks + n_tokens % 4;
    if (!sel && n_sel_blocks == a.nb)
        a.n_cells = n_tokens;      // every block kept: cells are 0..n-1
    a.n_split = (int32_t)n_splits(a.n_cells);
    a.kv_heads = d->kv_heads;
    a.scale = attn_scale(d);
    return a;
}

// The splits hold the chosen blocks' cells and the merge adds the <= 3 tail
// cells: 4K cells fill whole workgroups (2 x 128 16-cell splits in the decode
// attention, 2 x 32 64-cell iterations per sequence in the batch), where 4K +
// tail needs one more per KV head and, on a full chip, a second round for it.
void fold_tail(AttendArgs &a, int32_t n_tokens)
{
    if (a.n_sel_blocks > 0 && n_tokens % 4 != 0) {
        a.n_cells = 4 * a.n_sel_blocks;
        a.n_tail = n_tokens % 4;
        a.n_split = (int32_t)n_splits(a.n_cells);
    }
}

// Stage 4 launch shared by qsa_gather_attend and qsa_decode_step.
qsa_status do_attend(const qsa_layer_desc *d, const qsa_layer_cache *c, int32_t n_tokens,
                     const int32_t *sel, int32_t n_sel_blocks, const float *q, float *out,
                     float *part, hipStream_t stream)
{
    AttendArgs a = attend_args(d, c, n_tokens, sel, n_sel_blocks, q, out, part);
    fold_tail(a, n_tokens);
    hipError_t e = launch_attend(a, d->head_dim, d->q_heads / d->kv_heads, stream);
    if (e != hipSuccess)
        return hip_fail(e, "attend");
    return QSA_OK;
}

// Stage 1 arguments: append n_new rows (consecutive in their sources) at
// pos, then pool blocks [b0, b1).  rows may be null (no append).
UpdateArgs update_args(const qsa_layer_desc *d, const qsa_layer_cache *c, const float *gamma,
                       const void *idx_rows, const uint16_t *k_rows, const uint16_t *v_rows,
                       int64_t pos, int32_t n_new, int32_t b0, int32_t b1)
{
    UpdateArgs u{};
    u.idx_k = c->idx_k;
    u.summary = c->summary;
    u.k = c->k;
    u.v = c->v;
    u.new_idx_row = idx_rows;
    u.new_k_row = k_rows;
    u.new_v_row = v_rows;
    u.gamma = gamma;
    u.idx_row_words = d->idx_heads * d->idx_dim * elem_bytes(d->idx_dtype) / 4;
    u.kv_row_words = d->kv_heads * d->head_dim / 2;
    u.pos = pos;
    u.n_new = n_new;
    u.b0 = b0;
    u.nblk = b1 - b0;
    u.H = d->idx_heads;
    u.D = d->idx_dim;
    u.eps = (double)d->rms_eps;
    u.theta = (double)d->rope_theta;
    return u;
}

// Entries T of each R-block tile list for nb blocks and k kept: a tile can
// hide a winner from the lists only if it holds T or more of the k winners.
// With winners spread at random, a tile holds X ~ Poisson(R k / nb) of them;
// T is the shortest of R/8, R/4, R/2 (at most 32) for which the expected
// number of such tiles, ntiles P(X >= T), is below 1e-4, within what the
// fast path of the top-k holds.  (Failing the check costs time, not
// exactness: the top-k then runs over every key.)
int32_t list_len(int32_t tile_rows, int64_t nb, int32_t k)
{
    const int32_t base = tile_rows / kListDiv;
    if (nb <= 0)
        return base;
    const int64_t ntiles = (nb + tile_rows - 1) / tile_rows;
    const double lam = (double)tile_rows * (double)(k < nb ? k : nb) / (double)nb;
    int32_t best = base;
    for (int32_t T = base; T <= 32 && T <= tile_rows / 2; T *= 2) {
        if (!sel::fits_fast((int32_t)ntiles, T))
            break;
        best = T;
        double term = exp(-lam);            // P(X = x), x = 0 ..
        for (int32_t x = 0; x < T; ++x)
            term *= lam / (double)(x + 1);
        double tail = 0.0;                  // P(X >= T)
        for (int32_t x = T; x < T + 200 && term > 0.0; ++x) {
            tail += term;
            term *= lam / (double)(x + 1);
        }
        if ((double)ntiles * tail < 1e-4)
            break;
    }
    return best;
}

// Top-k arguments over the keys and tile lists (T entries each) already in
// the workspace.
SelectArgs select_args(char *ws, const WsLayout &L, int32_t nb, int32_t k, int32_t tile_rows,
                       int32_t list_t, int32_t *sel)
{
    SelectArgs s{};
    s.keys = (const uint32_t *)(ws + L.keys);
    s.lists = (const uint64_t *)(ws + L.lists);
    s.sel = sel;
    s.nb = nb;
    s.k = k;
    s.ntiles = (nb + tile_rows - 1) / tile_rows;
    s.T = list_t;
    return s;
}

qsa_status do_select(char *ws, const WsLayout &L, int32_t nb, int32_t k, int32_t tile_rows,
                     int32_t *sel, hipStream_t stream)
{
    hipError_t e = launch_select(select_args(ws, L, nb, k, tile_rows, tile_rows / kListDiv, sel),
                                 stream);
    if (e != hipSuccess)
        return hip_fail(e, "select");
    return QSA_OK;
}

}  // namespace

extern "C" {

size_t qsa_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity)
{
    if (check_desc(desc) != QSA_OK || capacity < 4 || capacity % 4 != 0 || capacity > (1 << 21))
        return 0;
    return decode_layout(desc, capacity).total;
}

void qsa_state_invalidate(qsa_seq_state *st, int32_t pos)
{
    if (!st)
        return;
    if (pos < 0)
        pos = 0;
    const int32_t b = pos / 4;
    if (st->n_valid_blocks > b)
        st->n_valid_blocks = b;
}

void qsa_state_truncate(qsa_seq_state *st, int32_t pos)
{
    if (!st)
        return;
    if (pos < 0)
        pos = 0;
    if (st->n_tokens > pos)
        st->n_tokens = pos;
    qsa_state_invalidate(st, pos);
}

qsa_status qsa_cache_update(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                            const float *gamma, int32_t blk_begin, int32_t blk_end,
                            hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, true, true, false)) != QSA_OK)
        return s;
    if (!gamma)
        return fail(QSA_ERR_ARG, "gamma is NULL");
    if (blk_begin < 0 || blk_end < blk_begin || blk_end > cache->capacity / 4)
        return fail(QSA_ERR_ARG, "block range [%d, %d) outside [0, %d]", blk_begin, blk_end,
                    cache->capacity / 4);
    if (blk_end == blk_begin)
        return ok();
    const UpdateArgs a =
        update_args(desc, cache, gamma, nullptr, nullptr, nullptr, 0, 0, blk_begin, blk_end);
    hipError_t e = launch_update(a, desc->idx_dtype == QSA_F16, stream);
    if (e != hipSuccess)
        return hip_fail(e, "cache_update");
    return ok();
}

qsa_status qsa_index_score(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                           int32_t n_blocks, const float *q_idx, const float *w, float *scores,
                           hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, false, true, false)) != QSA_OK)
        return s;
    if (n_blocks < 0 || n_blocks > cache->capacity / 4)
        return fail(QSA_ERR_ARG, "n_blocks %d outside [0, %d]", n_blocks, cache->capacity / 4);
    if (!q_idx || !w || !scores)
        return fail(QSA_ERR_ARG, "q_idx / w / scores is NULL");
    if (!aligned(q_idx, 16))
        return fail(QSA_ERR_ARG, "q_idx must be 16-byte aligned");
    if (n_blocks == 0)
        return ok();
    ScoreArgs a{};
    a.summary = cache->summary;
    a.q = q_idx;
    a.w = w;
    a.scores = scores;
    a.nb = n_blocks;
    a.D = desc->idx_dim;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    hipError_t e = launch_score(a, desc->idx_dtype == QSA_F16, rowb, stream);
    if (e != hipSuccess)
        return hip_fail(e, "index_score");
    return ok();
}

qsa_status qsa_topk_blocks(const float *scores, int32_t n_blocks, int32_t k_blocks, int32_t *sel,
                           void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (n_blocks < 0 || n_blocks > (1 << 19) || k_blocks < 1)
        return fail(QSA_ERR_ARG, "n_blocks %d / k_blocks %d out of range", n_blocks, k_blocks);
    if ((n_blocks > 0 && !scores) || !sel)
        return fail(QSA_ERR_ARG, "scores / sel is NULL");
    if (n_blocks == 0)
        return ok();
    if (n_blocks <= k_blocks) {
        hipError_t e = launch_iota(sel, n_blocks, stream);
        return e == hipSuccess ? ok() : hip_fail(e, "topk_blocks");
    }
    const WsLayout L = ws_layout(n_blocks, 0, 0);
    qsa_status st = check_ws(ws, ws_bytes, L.total);
    if (st != QSA_OK)
        return st;
    char *w = (char *)ws;
    hipError_t e = launch_keys(scores, n_blocks, (uint32_t *)(w + L.keys),
                               (uint64_t *)(w + L.lists), stream);
    if (e != hipSuccess)
        return hip_fail(e, "topk_blocks");
    st = do_select(w, L, n_blocks, k_blocks, kKeysTile, sel, stream);
    return st == QSA_OK ? ok() : st;
}

qsa_status qsa_gather_attend(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                             int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                             const float *q, float *out, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, false, false, true)) != QSA_OK)
        return s;
    const int32_t nb = n_tokens / 4;
    const int32_t K = desc->top_k_tokens / 4;
    if (n_tokens < 1 || n_tokens > cache->capacity)
        return fail(QSA_ERR_ARG, "n_tokens %d outside [1, %d]", n_tokens, cache->capacity);
    if (n_sel_blocks < 0 || n_sel_blocks > nb || n_sel_blocks > K)
        return fail(QSA_ERR_ARG, "n_sel_blocks %d outside [0, min(%d, %d)]", n_sel_blocks, K, nb);
    if (!sel && n_sel_blocks != nb)
        return fail(QSA_ERR_ARG, "sel may be NULL only when every block is kept");
    if (n_sel_blocks == 0 && n_tokens % 4 == 0)
        return fail(QSA_ERR_ARG, "no cell to attend (no block and no tail cell)");
    if (!q || !out)
        return fail(QSA_ERR_ARG, "q / out is NULL");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "q / out must be 16-byte aligned");
    const WsLayout L = decode_layout(desc, cache->capacity);
    if ((s = check_ws(ws, ws_bytes, L.total)) != QSA_OK)
        return s;
    s = do_attend(desc, cache, n_tokens, sel, n_sel_blocks, q, out,
                  (float *)((char *)ws + L.part), stream);
    return s == QSA_OK ? ok() : s;
}

// How a decode step over nb completed blocks selects: the histogram path
// (score pass + k_decode.hip) when the shapes fit it, with ns splits per KV
// head, a fresh epoch and the default window.
struct DecodePlan {
    bool hist_path;
    int64_t ns;
    uint64_t epoch;
    float def_k;
};

DecodePlan decode_plan(const qsa_layer_desc *desc, int32_t nb)
{
    const int32_t K = desc->top_k_tokens / 4;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const int tile_rows = score_tile_rows(desc->idx_dtype == QSA_F16, rowb);
    const int32_t list_t = list_len(tile_rows, nb, K);
    const int64_t ntiles = ((int64_t)nb + tile_rows - 1) / tile_rows;
    const int G = desc->q_heads / desc->kv_heads;
    DecodePlan P{};
    P.ns = device_cus() / desc->kv_heads;
    if (P.ns > kDecodeMaxSplits)
        P.ns = kDecodeMaxSplits;
    if (P.ns > ntiles)
        P.ns = ntiles;
    P.hist_path = nb > K && P.ns >= 1 && ((ntiles + P.ns - 1) / P.ns) * list_t <= kDecodeThreads &&
                  (int64_t)desc->kv_heads * P.ns <= kDecodeThreads && decode_fits(nb, desc->head_dim, G);
    P.epoch = P.hist_path ? next_epoch() : 0;
    P.def_k = P.hist_path ? default_kappa(nb, K) : 0.0f;
    return P;
}

// The decode step's score pass: scores (optional), keys and tile lists when
// there is a selection, the histogram on the histogram path.
ScoreArgs decode_score_args(const qsa_layer_desc *desc, const qsa_layer_cache *cache, const WsLayout &L,
                            char *wsp, const DecodePlan &P, int32_t nb, bool need_select, const float *gamma,
                            const float *q_idx, const float *w, float *scores_out)
{
    const int32_t K = desc->top_k_tokens / 4;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const int tile_rows = score_tile_rows(desc->idx_dtype == QSA_F16, rowb);
    ScoreArgs a{};
    a.summary = cache->summary;
    a.q = q_idx;
    a.w = w;
    a.scores = scores_out;
    a.keys = need_select ? (uint32_t *)(wsp + L.keys) : nullptr;
    a.lists = need_select ? (uint64_t *)(wsp + L.lists) : nullptr;
    a.list_t = list_len(tile_rows, nb, K);
    a.nb = nb;
    a.D = desc->idx_dim;
    if (P.hist_path) {
        a.h.hist = (uint32_t *)(wsp + L.hist);
        a.h.bmax = (uint64_t *)(wsp + L.bmax);
        a.h.bminc = (uint64_t *)(wsp + L.bminc);
        a.h.last = (uint64_t *)(wsp + L.last);
        a.h.ctrl = wsp + L.ctrl;
        a.h.gamma = gamma;
        a.h.epoch = P.epoch;
        a.h.def_k = P.def_k;
        a.h.def_top = P.def_k + 2.5f;
    }
    return a;
}

qsa_status qsa_decode_step(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                           qsa_seq_state *st, const void *idx_k_row, const uint16_t *k_row,
                           const uint16_t *v_row, const float *gamma, const float *q_idx,
                           const float *w, const float *q, float *out, int32_t *sel_out,
                           float *scores_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, true, true, true)) != QSA_OK)
        return s;
    if (!st)
        return fail(QSA_ERR_ARG, "state is NULL");
    if (!idx_k_row || !k_row || !v_row || !gamma || !q_idx || !w || !q || !out)
        return fail(QSA_ERR_ARG, "an input or output pointer is NULL");
    if (!aligned(idx_k_row, 4) || !aligned(k_row, 4) || !aligned(v_row, 4) ||
        !aligned(q, 16) || !aligned(q_idx, 16))
        return fail(QSA_ERR_ARG,
                    "row pointers must be 4-byte aligned and q, q_idx 16-byte aligned");
    const int32_t pos = st->n_tokens;
    if (pos < 0 || pos >= cache->capacity)
        return fail(QSA_ERR_ARG, "position %d outside [0, %d)", pos, cache->capacity);
    if (st->n_valid_blocks < 0)
        return fail(QSA_ERR_ARG, "n_valid_blocks %d < 0", st->n_valid_blocks);
    const WsLayout L = decode_layout(desc, cache->capacity);
    if ((s = check_ws(ws, ws_bytes, L.total)) != QSA_OK)
        return s;

    const int32_t n = pos + 1;
    const int32_t nb = n / 4;
    const int32_t K = desc->top_k_tokens / 4;
    const int32_t b0 = st->n_valid_blocks < nb ? st->n_valid_blocks : nb;
    const bool need_select = nb > K;
    const int ebytes = elem_bytes(desc->idx_dtype);
    const int rowb = desc->idx_heads * desc->idx_dim * ebytes;
    char *wsp = (char *)ws;

    // 1. append + pool [b0, nb).  One new row (the usual decode step) is pooled
    //    by the score kernel's first workgroup; anything else runs on its own.
    const UpdateArgs u = update_args(desc, cache, gamma, idx_k_row, k_row, v_row, pos, 1, b0, nb);
    const bool score = nb > 0 && (need_select || scores_out);
    const bool fuse = score && u.nblk <= 1;
    hipError_t e;
    if (!fuse) {
        e = launch_update(u, desc->idx_dtype == QSA_F16, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step/update");
    }

    // 2. score every completed block (keys for the top-k).  With a selection
    //    the pass also fills the global histogram, from which the attention
    //    kernel selects (k_decode.hip) when the shapes fit it.
    const int tile_rows = score_tile_rows(desc->idx_dtype == QSA_F16, rowb);
    const int32_t list_t = list_len(tile_rows, nb, K);
    const int G = desc->q_heads / desc->kv_heads;
    const DecodePlan P = decode_plan(desc, nb);
    const bool hist_path = P.hist_path;
    const int64_t ns = P.ns;
    const uint64_t epoch = P.epoch;
    if (score) {
        ScoreArgs a = decode_score_args(desc, cache, L, wsp, P, nb, need_select, gamma, q_idx, w, scores_out);
        a.fuse = fuse ? 1 : 0;
        a.upd = u;
        e = launch_score(a, desc->idx_dtype == QSA_F16, rowb, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step/score");
    }

    // 3 + 4. top-k (every block is kept when nb <= K), gather + attend.
    float *part = (float *)(wsp + L.part);
    if (hist_path) {
        DecodeArgs da{};
        da.k = cache->k;
        da.v = cache->v;
        da.q = q;
        da.out = out;
        da.sel_out = sel_out;
        da.nb = nb;
        da.n_tail = n % 4;
        da.kv_heads = desc->kv_heads;
        da.k_blocks = K;
        da.scale = attn_scale(desc);
        da.sa = select_args(wsp, L, nb, K, tile_rows, list_t, nullptr);
        da.hist = (const uint32_t *)(wsp + L.hist);
        da.bmax = (const uint64_t *)(wsp + L.bmax);
        da.bminc = (const uint64_t *)(wsp + L.bminc);
        da.last = (const uint64_t *)(wsp + L.last);
        da.ctrl = wsp + L.ctrl;
        da.ns = (int32_t)ns;
        da.part = part;
        da.stage = (int32_t *)(wsp + L.stage);
        da.stage_n = (int32_t *)(wsp + L.stage_n);
        da.epoch = epoch;
        e = launch_decode_attend(da, desc->head_dim, G, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step/decode_attend");
    } else if (need_select) {
        SelectArgs sa = select_args(wsp, L, nb, K, tile_rows, list_t, sel_out);
        // fused: the splits hold the 4K chosen cells, the merge adds the tail
        AttendArgs aa = attend_args(desc, cache, n, nullptr, K, q, out, part);
        aa.n_cells = 4 * K;
        aa.n_tail = n % 4;
        aa.n_split = (int32_t)n_splits(aa.n_cells);
        if (sel::fits_fast(sa.ntiles, sa.T) &&
            (int64_t)aa.n_split * aa.kv_heads <= device_cus()) {
            e = launch_select_attend(aa, sa, desc->head_dim, G, stream);
            if (e != hipSuccess)
                return hip_fail(e, "decode_step/select_attend");
        } else {
            int32_t *dst = sel_out ? sel_out : (int32_t *)(wsp + L.sel);
            sa.sel = dst;
            e = launch_select(sa, stream);
            if (e != hipSuccess)
                return hip_fail(e, "decode_step/select");
            if ((s = do_attend(desc, cache, n, dst, K, q, out, part, stream)) != QSA_OK)
                return s;
        }
    } else {
        if (sel_out && nb > 0) {
            e = launch_iota(sel_out, nb, stream);
            if (e != hipSuccess)
                return hip_fail(e, "decode_step/iota");
        }
        if ((s = do_attend(desc, cache, n, nullptr, nb, q, out, part, stream)) != QSA_OK)
            return s;
    }

    st->n_tokens = n;
    st->n_valid_blocks = nb;
    return ok();
}

// ----------------------------------------------- decode step without allocation
// The workspace of qsa_decode_step_static: one array per device, held until
// the process ends.  Host code never uses the array's name as an address:
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current.
static __device__ __align__(256) unsigned char scratch[QSA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (its address looked up once).
qsa_status static_scratch(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "decode_step_static/hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ERR_UNSUPPORTED, "device %d beyond the %d the static workspace serves", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "decode_step_static/hipGetSymbolAddress");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QSA_OK;
}
}  // namespace

qsa_status qsa_decode_step_static(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                  qsa_seq_state *st, const void *idx_k_row, const uint16_t *k_row,
                                  const uint16_t *v_row, const float *gamma, const float *q_idx,
                                  const float *w, const float *q, float *out, int32_t *sel_out,
                                  float *scores_out, hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, true, true, true)) != QSA_OK)
        return s;
    const size_t need = decode_layout(desc, cache->capacity).total;
    if (need > (size_t)QSA_STATIC_SCRATCH_BYTES)
        return fail(QSA_ERR_WORKSPACE,
                    "this cache needs a %zu-byte workspace, above the static one's %zu bytes "
                    "(use qsa_decode_step with a workspace)",
                    need, (size_t)QSA_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((s = static_scratch(&ws)) != QSA_OK)
        return s;
    return qsa_decode_step(desc, cache, st, idx_k_row, k_row, v_row, gamma, q_idx, w, q, out, sel_out,
                           scores_out, ws, (size_t)QSA_STATIC_SCRATCH_BYTES, stream);
}

qsa_status qsa_decode_score(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                            const qsa_seq_state *st, const float *gamma, const float *q_idx,
                            const float *w, float *scores_out, void *ws, size_t ws_bytes,
                            hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, false, true, false)) != QSA_OK)
        return s;
    if (!st)
        return fail(QSA_ERR_ARG, "state is NULL");
    if (!gamma || !q_idx || !w)
        return fail(QSA_ERR_ARG, "gamma / q_idx / w is NULL");
    if (!aligned(q_idx, 16))
        return fail(QSA_ERR_ARG, "q_idx must be 16-byte aligned");
    const int32_t n = st->n_tokens;
    if (n < 0 || n > cache->capacity)
        return fail(QSA_ERR_ARG, "n_tokens %d outside [0, %d]", n, cache->capacity);
    const WsLayout L = decode_layout(desc, cache->capacity);
    if ((s = check_ws(ws, ws_bytes, L.total)) != QSA_OK)
        return s;
    const int32_t nb = n / 4;
    const int32_t K = desc->top_k_tokens / 4;
    if (nb == 0 || (nb <= K && !scores_out))
        return ok();
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const DecodePlan P = decode_plan(desc, nb);
    const ScoreArgs a = decode_score_args(desc, cache, L, (char *)ws, P, nb, nb > K, gamma, q_idx, w, scores_out);
    const hipError_t e = launch_score(a, desc->idx_dtype == QSA_F16, rowb, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode_score");
    return ok();
}

size_t qsa_batch_workspace_bytes(const qsa_layer_desc *desc, int32_t n_seq,
                                 const int32_t *capacities)
{
    if (check_desc(desc) != QSA_OK || n_seq < 1 || n_seq > QSA_MAX_BATCH || !capacities)
        return 0;
    size_t total = 0;
    for (int32_t i = 0; i < n_seq; ++i) {
        const int32_t c = capacities[i];
        if (c < 4 || c % 4 != 0 || c > (1 << 21))
            return 0;
        total += align256(decode_layout(desc, c).total);
    }
    return total;
}

qsa_status qsa_decode_step_batch(const qsa_layer_desc *desc, int32_t n_seq,
                                 const qsa_layer_cache *caches, qsa_seq_state *states,
                                 const qsa_seq_io *io, const float *gamma, void *ws,
                                 size_t ws_bytes, hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK)
        return s;
    if (n_seq < 1 || n_seq > QSA_MAX_BATCH)
        return fail(QSA_ERR_ARG, "n_seq %d outside [1, %d]", n_seq, QSA_MAX_BATCH);
    if (!caches || !states || !io || !gamma)
        return fail(QSA_ERR_ARG, "caches / states / io / gamma is NULL");
    size_t need = 0;
    for (int32_t i = 0; i < n_seq; ++i) {
        if ((s = check_cache(&caches[i], true, true, true)) != QSA_OK) {
            char why[sizeof(tl_err)];
            snprintf(why, sizeof(why), "%s", tl_err);
            return fail(s, "sequence %d: %s", i, why);
        }
        const qsa_seq_io &x = io[i];
        if (!x.idx_k_row || !x.k_row || !x.v_row || !x.q_idx || !x.w || !x.q || !x.out)
            return fail(QSA_ERR_ARG, "sequence %d: an input or output pointer is NULL", i);
        if (!aligned(x.idx_k_row, 4) || !aligned(x.k_row, 4) || !aligned(x.v_row, 4) ||
            !aligned(x.q, 16) || !aligned(x.q_idx, 16))
            return fail(QSA_ERR_ARG, "sequence %d: misaligned pointer", i);
        const int32_t pos = states[i].n_tokens;
        if (pos < 0 || pos >= caches[i].capacity)
            return fail(QSA_ERR_ARG, "sequence %d: position %d outside [0, %d)", i, pos,
                        caches[i].capacity);
        if (states[i].n_valid_blocks < 0)
            return fail(QSA_ERR_ARG, "sequence %d: n_valid_blocks < 0", i);
        need += align256(decode_layout(desc, caches[i].capacity).total);
    }
    if ((s = check_ws(ws, ws_bytes, need)) != QSA_OK)
        return s;

    const int32_t K = desc->top_k_tokens / 4;
    const bool f16 = desc->idx_dtype == QSA_F16;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const int tile_rows = score_tile_rows(f16, rowb);
    const int G = desc->q_heads / desc->kv_heads;
    ScoreBatchArgs sb{};
    SelectBatchArgs selb{};
    AttendBatchArgs ab{};
    sb.n = selb.n = ab.n = n_seq;
    size_t off = 0;
    hipError_t e;
    for (int32_t i = 0; i < n_seq; ++i) {
        const qsa_layer_cache *c = &caches[i];
        const qsa_seq_io &x = io[i];
        const WsLayout L = decode_layout(desc, c->capacity);
        char *wsp = (char *)ws + off;
        off += align256(L.total);
        const int32_t pos = states[i].n_tokens;
        const int32_t n = pos + 1, nb = n / 4;
        const int32_t b0 = states[i].n_valid_blocks < nb ? states[i].n_valid_blocks : nb;
        const bool need_select = nb > K;

        const UpdateArgs u =
            update_args(desc, c, gamma, x.idx_k_row, x.k_row, x.v_row, pos, 1, b0, nb);
        const bool fuse = u.nblk <= 1;
        if (!fuse) {   // a rebuild after invalidation: its own launch first
            e = launch_update(u, f16, stream);
            if (e != hipSuccess)
                return hip_fail(e, "decode_step_batch/update");
        }
        ScoreArgs &a = sb.seq[i];
        a.summary = c->summary;
        a.q = x.q_idx;
        a.w = x.w;
        a.scores = x.scores_out;
        a.keys = need_select ? (uint32_t *)(wsp + L.keys) : nullptr;
        a.lists = need_select ? (uint64_t *)(wsp + L.lists) : nullptr;
        a.list_t = list_len(tile_rows, nb, K);
        // kept-everything sequences only run the prologue (and their scores when asked)
        a.nb = need_select || x.scores_out ? nb : 0;
        a.D = desc->idx_dim;
        a.fuse = fuse ? 1 : 0;
        a.upd = u;

        int32_t *sel = need_select ? (x.sel_out ? x.sel_out : (int32_t *)(wsp + L.sel)) : x.sel_out;
        selb.seq[i] = select_args(wsp, L, nb, K, tile_rows, a.list_t, sel);
        ab.seq[i] = attend_args(desc, c, n, need_select ? sel : nullptr, need_select ? K : nb,
                                x.q, x.out, (float *)(wsp + L.part));
        fold_tail(ab.seq[i], n);
    }
    e = launch_score_batch(sb, f16, rowb, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode_step_batch/score");
    e = launch_select_batch(selb, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode_step_batch/select");
    e = launch_attend_batch(ab, desc->head_dim, G, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode_step_batch/attend");
    for (int32_t i = 0; i < n_seq; ++i) {
        states[i].n_tokens += 1;
        states[i].n_valid_blocks = states[i].n_tokens / 4;
    }
    return ok();
}

size_t qsa_multi_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity, int32_t n_q)
{
    if (check_desc(desc) != QSA_OK || capacity < 4 || capacity % 4 != 0 || capacity > (1 << 21) ||
        n_q < 1 || n_q > QSA_MAX_MULTI)
        return 0;
    return (size_t)n_q * align256(decode_layout(desc, capacity).total);
}

qsa_status qsa_decode_step_multi(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                 qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                                 const uint16_t *k_rows, const uint16_t *v_rows,
                                 const float *gamma, const float *q_idx, const float *w,
                                 const float *q, float *out, int32_t *sel_out, float *scores_out,
                                 void *ws, size_t ws_bytes, hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, true, true, true)) != QSA_OK)
        return s;
    if (!st)
        return fail(QSA_ERR_ARG, "state is NULL");
    if (n_q < 1 || n_q > QSA_MAX_MULTI)
        return fail(QSA_ERR_ARG, "n_q %d outside [1, %d]", n_q, QSA_MAX_MULTI);
    if (!idx_k_rows || !k_rows || !v_rows || !gamma || !q_idx || !w || !q || !out)
        return fail(QSA_ERR_ARG, "an input or output pointer is NULL");
    if (!aligned(idx_k_rows, 16) || !aligned(k_rows, 16) || !aligned(v_rows, 16) ||
        !aligned(q_idx, 16) || !aligned(q, 16) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "row, q_idx, q or out pointer not 16-byte aligned");
    const int32_t n0 = st->n_tokens;
    if (n0 < 0 || (int64_t)n0 + n_q > cache->capacity)
        return fail(QSA_ERR_ARG, "positions [%d, %lld) outside [0, %d)", n0,
                    (long long)n0 + n_q, cache->capacity);
    if (st->n_valid_blocks < 0)
        return fail(QSA_ERR_ARG, "n_valid_blocks < 0");
    const WsLayout L = decode_layout(desc, cache->capacity);
    const size_t slot = align256(L.total);
    if ((s = check_ws(ws, ws_bytes, (size_t)n_q * slot)) != QSA_OK)
        return s;

    const int32_t K = desc->top_k_tokens / 4;
    const int32_t n_end = n0 + n_q, nb_last = n_end / 4;
    const bool f16 = desc->idx_dtype == QSA_F16;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const int G = desc->q_heads / desc->kv_heads;
    const int qk = desc->idx_heads * desc->idx_dim;
    const int64_t qa = (int64_t)desc->q_heads * desc->head_dim;
    const int32_t b0 = st->n_valid_blocks < nb_last ? st->n_valid_blocks : nb_last;
    const bool any_select = nb_last > K;       // the last query sees the most blocks

    // 1. append the n_q rows, pool [b0, nb_last): inside the score kernel's
    //    first workgroup when at most one row is new, else in its own launch
    const UpdateArgs u =
        update_args(desc, cache, gamma, idx_k_rows, k_rows, v_rows, n0, n_q, b0, nb_last);
    const bool score = nb_last > 0 && (any_select || scores_out);
    const bool fuse = score && u.nblk <= 1;
    hipError_t e;
    if (!fuse) {
        e = launch_update(u, f16, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step_multi/update");
    }

    // 2. one pass over the summaries for every query
    const int tile_rows = score_tile_rows(f16, rowb);
    SelectBatchArgs selb{};
    AttendBatchArgs ab{};
    selb.n = ab.n = n_q;
    ScoreMultiArgs sm{};
    sm.summary = cache->summary;
    sm.nb = nb_last;
    sm.D = desc->idx_dim;
    sm.fuse = fuse ? 1 : 0;
    sm.upd = u;
    sm.scores = scores_out;
    sm.ld_scores = nb_last;
    sm.list_t = list_len(tile_rows, nb_last, K);   // one list length for every query
    for (int32_t i = 0; i < n_q; ++i) {
        char *wsp = (char *)ws + (size_t)i * slot;
        const int32_t n = n0 + i + 1, nb = n / 4;
        const bool need_select = nb > K;
        sm.nbq[i] = nb;
        sm.q[i] = q_idx + (size_t)i * qk;
        sm.w[i] = w + (size_t)i * desc->idx_heads;
        sm.keys[i] = need_select ? (uint32_t *)(wsp + L.keys) : nullptr;
        sm.lists[i] = need_select ? (uint64_t *)(wsp + L.lists) : nullptr;
        int32_t *sel = sel_out ? sel_out + (size_t)i * K : (int32_t *)(wsp + L.sel);
        selb.seq[i] = select_args(wsp, L, nb, K, tile_rows, sm.list_t,
                                  need_select || sel_out ? sel : nullptr);
        selb.seq[i].pad_to = sel_out ? K : 0;
        ab.seq[i] = attend_args(desc, cache, n, need_select ? sel : nullptr, need_select ? K : nb,
                                q + (size_t)i * qa, out + (size_t)i * qa,
                                (float *)(wsp + L.part));
        fold_tail(ab.seq[i], n);
    }
    if (score) {
        e = launch_score_multi(sm, n_q, f16, rowb, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step_multi/score");
    }

    // 3. per-query top-k (one workgroup per query), 4. per-query attention
    if (any_select || sel_out) {
        e = launch_select_batch(selb, stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode_step_multi/select");
    }
    e = launch_attend_batch(ab, desc->head_dim, G, stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode_step_multi/attend");
    st->n_tokens = n_end;
    st->n_valid_blocks = nb_last;
    return ok();
}

size_t qsa_chunk_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity, int32_t n_q)
{
    if (check_desc(desc) != QSA_OK || capacity < 4 || capacity % 4 != 0 || capacity > (1 << 21) ||
        n_q < 1 || n_q > QSA_MAX_CHUNK)
        return 0;
    const size_t chunk = chunk_layout(desc, capacity, n_q).total;
    if (n_q > QSA_MAX_MULTI)
        return chunk;
    const size_t multi = qsa_multi_workspace_bytes(desc, capacity, n_q);
    return multi > chunk ? multi : chunk;
}

namespace {
qsa_status chunk_step(const qsa_layer_desc *desc, const qsa_layer_cache *cache, qsa_seq_state *st,
                      int32_t n_q, const void *idx_k_rows, const uint16_t *k_rows, const uint16_t *v_rows,
                      const float *gamma, const float *q_idx, const float *w, const float *q, float *out,
                      int32_t *sel_out, float *scores_out, void *ws, size_t ws_bytes, hipStream_t stream,
                      bool grouped)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, true, true, true)) != QSA_OK)
        return s;
    if (!st)
        return fail(QSA_ERR_ARG, "state is NULL");
    if (n_q < 1 || n_q > QSA_MAX_CHUNK)
        return fail(QSA_ERR_ARG, "n_q %d outside [1, %d]", n_q, QSA_MAX_CHUNK);
    if (!idx_k_rows || !k_rows || !v_rows || !gamma || !q_idx || !w || !q || !out)
        return fail(QSA_ERR_ARG, "an input or output pointer is NULL");
    if (!aligned(idx_k_rows, 16) || !aligned(k_rows, 16) || !aligned(v_rows, 16) ||
        !aligned(q_idx, 16) || !aligned(q, 16) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "row, q_idx, q or out pointer not 16-byte aligned");
    const int32_t n0 = st->n_tokens;
    if (n0 < 0 || (int64_t)n0 + n_q > cache->capacity)
        return fail(QSA_ERR_ARG, "positions [%d, %lld) outside [0, %d)", n0,
                    (long long)n0 + n_q, cache->capacity);
    if (st->n_valid_blocks < 0)
        return fail(QSA_ERR_ARG, "n_valid_blocks < 0");
    // a few tokens: one pass over the summaries scores them all, without the
    // GEMM's query preparation and its keys matrix
    if (n_q <= QSA_MAX_MULTI)
        return qsa_decode_step_multi(desc, cache, st, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx,
                                     w, q, out, sel_out, scores_out, ws, ws_bytes, stream);
    const ChunkLayout L = chunk_layout(desc, cache->capacity, n_q);
    if ((s = check_ws(ws, ws_bytes, L.total)) != QSA_OK)
        return s;

    const bool f16 = desc->idx_dtype == QSA_F16;
    const int rowb = desc->idx_heads * desc->idx_dim * elem_bytes(desc->idx_dtype);
    const int G = desc->q_heads / desc->kv_heads;
    const int32_t K = desc->top_k_tokens / 4;
    const int32_t n_end = n0 + n_q, nb_last = n_end / 4;
    char *wsp = (char *)ws;

    ChunkArgs c{};
    c.idx_k = cache->idx_k;
    c.summary = cache->summary;
    c.k = cache->k;
    c.v = cache->v;
    c.idx_rows = idx_k_rows;
    c.k_rows = k_rows;
    c.v_rows = v_rows;
    c.idx_row_bytes = rowb;
    c.kv_row_bytes = desc->kv_heads * desc->head_dim * 2;
    c.q_idx = q_idx;
    c.w = w;
    c.q = q;
    c.out = out;
    c.sel_out = sel_out;
    c.scores_out = scores_out;
    c.qhl = (_Float16 *)(wsp + L.qhl);
    c.qscale = (float *)(wsp + L.qscale);
    c.keys = (uint32_t *)(wsp + L.keys);
    c.sel = (int32_t *)(wsp + L.sel);
    c.part = (float *)(wsp + L.part);
    c.ldk = ((int64_t)nb_last + 3) / 4 * 4;
    c.n0 = n0;
    c.n_q = n_q;
    c.nb_last = nb_last;
    c.kb = K;
    c.H = desc->idx_heads;
    c.D = desc->idx_dim;
    c.kv_heads = desc->kv_heads;
    c.scale = attn_scale(desc);
    // few queries: split each query's iterations of 64 cells so that the
    // chip is still filled, every split getting at least one
    const int64_t units = (int64_t)n_q * desc->kv_heads;
    const int64_t max_it = (4 * (int64_t)K + 3 + kUnitCells - 1) / kUnitCells;
    int64_t ns = units >= kChunkWgTarget ? 1 : (kChunkWgTarget + units - 1) / units;
    ns = ns < max_it ? ns : max_it;
    ns = ns < kChunkMaxSplits ? ns : kChunkMaxSplits;
    ns = (max_it + (max_it + ns - 1) / ns - 1) / ((max_it + ns - 1) / ns);   // no split left empty
    c.n_split = (int32_t)ns;
    if (grouped) {
        const int qg = union_group(desc, nb_last);
        if (qg < 1)
            return fail(QSA_ERR_UNSUPPORTED, "no grouped-union group fits these shapes");
        c.union_q = qg;
        c.ucap = qg * K;
        c.uni = (int32_t *)(wsp + L.uni);
        c.umask = (uint32_t *)(wsp + L.umask);
        c.ucount = (int32_t *)(wsp + L.ucount);
    }

    hipError_t e = launch_chunk_append(c, stream);
    if (e != hipSuccess)
        return hip_fail(e, "chunk_step/append");
    const int32_t b0 = st->n_valid_blocks < nb_last ? st->n_valid_blocks : nb_last;
    if (nb_last > b0) {
        const UpdateArgs u =
            update_args(desc, cache, gamma, nullptr, nullptr, nullptr, 0, 0, b0, nb_last);
        e = launch_update(u, f16, stream);
        if (e != hipSuccess)
            return hip_fail(e, "chunk_step/pool");
    }
    e = launch_chunk_rest(c, f16, desc->head_dim, G, stream);
    if (e != hipSuccess)
        return hip_fail(e, "chunk_step");
    st->n_tokens = n_end;
    st->n_valid_blocks = nb_last;
    return ok();
}
}  // namespace

qsa_status qsa_chunk_step(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                          qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                          const uint16_t *k_rows, const uint16_t *v_rows, const float *gamma,
                          const float *q_idx, const float *w, const float *q, float *out,
                          int32_t *sel_out, float *scores_out, void *ws, size_t ws_bytes,
                          hipStream_t stream)
{
    return chunk_step(desc, cache, st, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx, w, q, out, sel_out,
                      scores_out, ws, ws_bytes, stream, false);
}

qsa_status qsa_chunk_step_grouped(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                  qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                                  const uint16_t *k_rows, const uint16_t *v_rows, const float *gamma,
                                  const float *q_idx, const float *w, const float *q, float *out,
                                  int32_t *sel_out, float *scores_out, void *ws, size_t ws_bytes,
                                  hipStream_t stream)
{
    return chunk_step(desc, cache, st, n_q, idx_k_rows, k_rows, v_rows, gamma, q_idx, w, q, out, sel_out,
                      scores_out, ws, ws_bytes, stream, true);
}

size_t qsa_ablation_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity)
{
    if (check_desc(desc) != QSA_OK || capacity < 4 || capacity % 4 != 0 || capacity > (1 << 21))
        return 0;
    const int32_t nb = capacity / 4;
    const int G = desc->q_heads / desc->kv_heads;
    // qsa_attend_masked: the block bitmap, then the split partials
    const size_t masked = align256(sizeof(uint32_t) * (size_t)((nb + 31) / 32)) +
                          align256(sizeof(float) * (size_t)desc->kv_heads * kMaskedMaxSplits *
                                   part_stride(G, desc->head_dim));
    // qsa_topk_cells: the expanded scores, then the keys and tile lists of the cells
    const size_t cells = align256(sizeof(float) * 4 * (size_t)nb) + ws_layout(4 * (int64_t)nb, 0, 0).total;
    return masked > cells ? masked : cells;
}

qsa_status qsa_topk_cells(const float *block_scores, int32_t n_tokens, int32_t top_k_tokens,
                          int32_t *cells, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (n_tokens < 1 || n_tokens / 4 > (1 << 17) || top_k_tokens < 4 || top_k_tokens % 4 != 0)
        return fail(QSA_ERR_ARG, "n_tokens %d / top_k_tokens %d out of range", n_tokens, top_k_tokens);
    const int32_t nb = n_tokens / 4, tail = n_tokens % 4;
    if ((nb > 0 && !block_scores) || !cells)
        return fail(QSA_ERR_ARG, "block_scores / cells is NULL");
    const size_t off = align256(sizeof(float) * 4 * (size_t)nb);
    const WsLayout L = ws_layout(4 * (int64_t)nb, 0, 0);
    qsa_status st = check_ws(ws, ws_bytes, off + L.total);
    if (st != QSA_OK)
        return st;
    hipError_t e = hipSuccess;
    const int32_t nc = 4 * nb;
    int32_t kept = nc;
    if (nc > top_k_tokens) {
        char *w = (char *)ws;
        float *cs = (float *)w;
        e = launch_expand_cells(block_scores, nb, cs, stream);
        if (e == hipSuccess)
            e = launch_keys(cs, nc, (uint32_t *)(w + off + L.keys), (uint64_t *)(w + off + L.lists),
                            stream);
        if (e == hipSuccess)
            e = launch_select(select_args(w + off, L, nc, top_k_tokens, kKeysTile,
                                          kKeysTile / kListDiv, cells),
                              stream);
        kept = top_k_tokens;
    } else if (nc > 0) {
        e = launch_iota(cells, nc, stream);
    }
    if (e == hipSuccess && tail > 0)
        e = launch_tail_cells(cells, kept, nb, tail, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "topk_cells");
}

qsa_status qsa_attend_masked(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                             int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                             const float *q, float *out, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK || (s = check_cache(cache, false, false, true)) != QSA_OK)
        return s;
    const int32_t nb = n_tokens / 4;
    if (n_tokens < 1 || n_tokens > cache->capacity)
        return fail(QSA_ERR_ARG, "n_tokens %d outside [1, %d]", n_tokens, cache->capacity);
    if (n_sel_blocks < 0 || n_sel_blocks > nb || (n_sel_blocks > 0 && !sel))
        return fail(QSA_ERR_ARG, "n_sel_blocks %d outside [0, %d] or sel NULL", n_sel_blocks, nb);
    if (n_sel_blocks == 0 && n_tokens % 4 == 0)
        return fail(QSA_ERR_ARG, "no cell to attend (no block and no tail cell)");
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "q / out NULL or not 16-byte aligned");
    const size_t need = qsa_ablation_workspace_bytes(desc, cache->capacity);
    if ((s = check_ws(ws, ws_bytes, need)) != QSA_OK)
        return s;
    MaskedArgs m{};
    m.k = cache->k;
    m.v = cache->v;
    m.sel = sel;
    m.q = q;
    m.out = out;
    m.bitmap = (uint32_t *)ws;
    m.part = (float *)((char *)ws + align256(sizeof(uint32_t) * (size_t)((cache->capacity / 4 + 31) / 32)));
    m.n_tokens = n_tokens;
    m.n_sel_blocks = n_sel_blocks;
    m.kv_heads = desc->kv_heads;
    m.scale = attn_scale(desc);
    hipError_t e = launch_masked_attend(m, desc->head_dim, desc->q_heads / desc->kv_heads, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "attend_masked");
}

qsa_status qsa_q8_0_quantize(const uint16_t *x, int64_t n_values, int8_t *codes, uint16_t *scales,
                             hipStream_t stream)
{
    if (n_values < 0 || n_values % 32 != 0)
        return fail(QSA_ERR_ARG, "n_values %lld is not a non-negative multiple of 32",
                    (long long)n_values);
    if (n_values == 0)
        return ok();
    if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2))
        return fail(QSA_ERR_ARG, "x / codes / scales NULL or misaligned");
    hipError_t e = launch_q8_0_quantize(x, n_values / 32, codes, scales, stream);
    if (e != hipSuccess)
        return hip_fail(e, "q8_0 quantize");
    return ok();
}

qsa_status qsa_gather_attend_q8_0(const qsa_layer_desc *desc, const qsa_kv_q8_0 *kv,
                                  int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                                  const float *q, float *out, void *ws, size_t ws_bytes,
                                  hipStream_t stream)
{
    qsa_status s;
    if ((s = check_desc(desc)) != QSA_OK)
        return s;
    if (!kv)
        return fail(QSA_ERR_ARG, "kv is NULL");
    if (kv->capacity < 4 || kv->capacity % 4 != 0 || kv->capacity > (1 << 21))
        return fail(QSA_ERR_ARG, "capacity must be a positive multiple of 4, <= 2^21 (got %d)",
                    kv->capacity);
    if (!kv->k_codes || !kv->v_codes || !kv->k_scales || !kv->v_scales ||
        !aligned(kv->k_codes, 16) || !aligned(kv->v_codes, 16) || !aligned(kv->k_scales, 16) ||
        !aligned(kv->v_scales, 16))
        return fail(QSA_ERR_ARG, "kv pointer NULL or not 16-byte aligned");
    const int32_t nb = n_tokens / 4;
    const int32_t K = desc->top_k_tokens / 4;
    if (n_tokens < 1 || n_tokens > kv->capacity)
        return fail(QSA_ERR_ARG, "n_tokens %d outside [1, %d]", n_tokens, kv->capacity);
    if (n_sel_blocks < 0 || n_sel_blocks > nb || n_sel_blocks > K)
        return fail(QSA_ERR_ARG, "n_sel_blocks %d outside [0, min(%d, %d)]", n_sel_blocks, K, nb);
    if (!sel && n_sel_blocks != nb)
        return fail(QSA_ERR_ARG, "sel may be NULL only when every block is kept");
    if (n_sel_blocks == 0 && n_tokens % 4 == 0)
        return fail(QSA_ERR_ARG, "no cell to attend (no block and no tail cell)");
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16))
        return fail(QSA_ERR_ARG, "q / out NULL or not 16-byte aligned");
    const WsLayout L = decode_layout(desc, kv->capacity);
    if ((s = check_ws(ws, ws_bytes, L.total)) != QSA_OK)
        return s;
    // the q8_0 planes stand in for the f16 rows; every other argument as in
    // the f16 gather (the merge adds the tail when blocks are chosen)
    qsa_layer_cache c{};
    c.k = (uint16_t *)kv->k_codes;
    c.v = (uint16_t *)kv->v_codes;
    c.capacity = kv->capacity;
    AttendArgs a = attend_args(desc, &c, n_tokens, sel, n_sel_blocks, q, out,
                               (float *)((char *)ws + L.part));
    fold_tail(a, n_tokens);
    hipError_t e = launch_attend_q8(a, kv->k_scales, kv->v_scales, desc->head_dim,
                                    desc->q_heads / desc->kv_heads, stream);
    if (e != hipSuccess)
        return hip_fail(e, "q8_0 attend");
    return ok();
}

const char *qsa_status_string(qsa_status s)
{
    switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape";
    case QSA_ERR_WORKSPACE: return "workspace missing or too small";
    case QSA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char *qsa_last_error(void) { return tl_err; }

}  // extern "C"
