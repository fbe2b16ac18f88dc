/*
 * qsa.h -- C ABI of the QSA (Qwen Sparse Attention) decode-step library for
 * AMD Instinct MI355X (gfx950).  Implemented in hand-written HIP kernels in
 * libqsa.so.
 *
 * Method source: post 10 by "ariera" on qiita.com, "第10回 EVO-X2（Ryzen AI Max+
 * 395 / 128GB）+ Qwen3.8-Flash-Next用のllama.cpp改造で長コンテキストのTGを高速化した話".
 * Sections cited by heading:
 *   "QSA indexer"                              -- pool / RMS norm / RoPE / score / top-k
 *   "incremental pooled-key cache（COMMON-004）" -- cache of completed-block summaries
 *   "selected QSA K/V gather（COMMON-005）"     -- attend over gathered K/V rows only
 *   "block-domain top-k（COMMON-006）実装は見送り" -- top-k on blocks, then tail cells
 *   "なぜFlash Attentionがcontext長に比例していたのか" -- at most 2048 + 4 - 1 cells
 *
 * One decode step of one layer, for the token at position n-1 (n tokens,
 * current one included), micro-block m = 4:
 *   N_b  = floor(n / 4) completed blocks, tail = n mod 4 cells;
 *   1. summary row b (b < N_b) = RoPE_{p=4b}( RMSNorm_gamma( mean of raw
 *      indexer-key rows 4b..4b+3 ) ), per indexer head, rounded once to the
 *      raw-key dtype; rows are cached and only [valid, N_b) are recomputed;
 *   2. s[b] = sum_h w[h] * <q_idx[h], summary[b][h]>  for b < N_b;
 *   3. the K_b = min(top_k_tokens / 4, N_b) blocks ranked first by
 *      (s descending, b ascending), returned as ascending ids;
 *   4. cells = {4b .. 4b+3 : b chosen} + {4 N_b .. n-1}  (4 K_b + tail <= 2051
 *      for top_k_tokens = 2048); for each query head h, with KV head
 *      g = floor(h * Hkv / Hq): out[h] = softmax_c(scale * <q[h], K[c][g]>) . V[c][g].
 *
 * Conventions
 *   - Every buffer is caller-owned.  Pointers marked DEVICE must point to
 *     device memory of the current HIP device, 16-byte aligned; HOST pointers
 *     are host memory.  The library never allocates, frees or synchronises.
 *   - Every call only enqueues work on `stream` and returns; results are
 *     valid when the stream reaches that point.  The host never reads device
 *     memory, so no call blocks.
 *   - Argument checks run before any launch.  On a failed check nothing is
 *     enqueued, no state is changed, and the status is QSA_ERR_ARG,
 *     QSA_ERR_UNSUPPORTED (shape outside the supported set) or
 *     QSA_ERR_WORKSPACE.  A launch failure (the HIP runtime refusing a
 *     launch, e.g. an invalid stream) returns QSA_ERR_HIP; kernels of the
 *     same call enqueued before the failing launch stay enqueued, and the
 *     sequence state is left unchanged.
 *     qsa_last_error() gives a thread-local description of the last failure.
 *   - Supported shapes: block = 4; idx_heads in {1, 4}; idx_dim in {64, 128};
 *     idx row (idx_heads * idx_dim * sizeof(dtype)) <= 1024 bytes;
 *     head_dim in {64, 128, 256}; q_heads = G * kv_heads with G in {1,2,4,8};
 *     top_k_tokens a positive
 *     multiple of 4, at most 16380; capacity a positive multiple of 4, at
 *     most 2^21 tokens (n_blocks of qsa_topk_blocks at most 2^19).
 *   - A workspace (DEVICE, 256-byte aligned, >= qsa_workspace_bytes) holds
 *     scratch.  Calls that share a workspace must be stream-ordered.  Its
 *     contents need no initialisation.  The decode step keeps a small region
 *     of it (a score histogram, qsa_decode_step below) cleared between calls
 *     and checks a tag before trusting it: a fresh or reused workspace only
 *     makes the first call take the slower exact path.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_ARG = -1,          /* null pointer, bad range, n > capacity, ... */
    QSA_ERR_UNSUPPORTED = -2,  /* shape outside the supported set above */
    QSA_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small */
    QSA_ERR_HIP = -4           /* a kernel launch failed */
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_F16 = 1 } qsa_dtype;

/* Per-layer constants (HOST struct, read during the call only). */
typedef struct {
    int32_t block;         /* micro-block size m; must be 4 */
    int32_t idx_heads;     /* H_i: indexer heads */
    int32_t idx_dim;       /* D_i: indexer head dim (even) */
    int32_t idx_dtype;     /* qsa_dtype of raw indexer keys AND of summaries */
    float rms_eps;         /* added to the mean square inside the root */
    float rope_theta;      /* RoPE base; frequency of pair j is theta^(-2j/D_i) */
    int32_t q_heads;       /* Hq */
    int32_t kv_heads;      /* Hkv */
    int32_t head_dim;      /* Dh */
    int32_t top_k_tokens;  /* indexer top-k in tokens; K = top_k_tokens / 4 blocks */
    float attn_scale;      /* logit scale; 0 means 1/sqrt(head_dim) */
} qsa_layer_desc;

/* One sequence x one layer cache (HOST struct of DEVICE pointers). */
typedef struct {
    void *idx_k;           /* DEVICE [capacity][H_i][D_i] idx_dtype; row t = position t */
    void *summary;         /* DEVICE [capacity/4][H_i][D_i] idx_dtype; row b = block b */
    uint16_t *k;           /* DEVICE [capacity][Hkv][Dh] binary16 bits; row t = position t */
    uint16_t *v;           /* DEVICE [capacity][Hkv][Dh] binary16 bits */
    int32_t capacity;      /* tokens */
} qsa_layer_cache;

/* Host-side sequence state: tokens in the cache and the summary watermark
 * (rows [0, n_valid_blocks) are trusted). */
typedef struct {
    int32_t n_tokens;
    int32_t n_valid_blocks;
} qsa_seq_state;

/* Scratch bytes needed by qsa_decode_step / qsa_gather_attend /
 * qsa_topk_blocks for any token count up to `capacity`.  Returns 0 for an
 * invalid or unsupported descriptor. */
size_t qsa_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity);

/* Diagnostics: a qsa_decode_step workspace holds, at this byte offset, a
 * 64-bit word whose low byte tells how the last decode step on it that
 * selected blocks chose them: QSA_PATH_HIST (the score histogram decided
 * exactly) or QSA_PATH_FULL (it could not, and the full top-k over every
 * block key ran).  The word is written by the device at the end of the step;
 * it is undefined before the first such step. */
#define QSA_DECODE_STATUS_OFFSET 8
#define QSA_PATH_HIST 1
#define QSA_PATH_FULL 2

/* State load or distrust from position `pos` [post 10, COMMON-004 section:
 * the cache is invalidated and rebuilt when next needed]:
 * n_valid_blocks = min(n_valid_blocks, floor(pos / 4)); tokens are kept.
 * HOST only; no device work.  Negative pos is treated as 0. */
void qsa_state_invalidate(qsa_seq_state *st, int32_t pos);

/* Sequence edit at `pos`: n_tokens = min(n_tokens, pos), then
 * qsa_state_invalidate(st, pos).  HOST only. */
void qsa_state_truncate(qsa_seq_state *st, int32_t pos);

/* Stage 1 [post 10, "QSA indexer", "incremental pooled-key cache
 * （COMMON-004）"]: (re)compute summary rows [blk_begin, blk_end) from raw
 * indexer-key rows 4*blk_begin .. 4*blk_end-1 already in cache->idx_k.
 * gamma: DEVICE fp32 [D_i].  Rows are independent; recomputing a range is
 * idempotent and bitwise deterministic.  Mean, norm and rotation are
 * evaluated in double (the RoPE angle at positions near 2^18 needs it) and
 * rounded once to the storage dtype.
 * Errors: ARG if 0 <= blk_begin <= blk_end <= capacity/4 fails or a needed
 * pointer is null.  An empty range enqueues nothing. */
qsa_status qsa_cache_update(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                            const float *gamma, int32_t blk_begin, int32_t blk_end,
                            hipStream_t stream);

/* Stage 2 [post 10, "QSA indexer"]: scores[b] = sum_h w[h] * sum_i
 * q_idx[h][i] * summary[b][h][i] for b < n_blocks, in fp32 (w folded into
 * q_idx once per call).  q_idx: DEVICE fp32 [H_i][D_i]; w: DEVICE fp32
 * [H_i]; scores: DEVICE fp32 [n_blocks].  n_blocks = 0 enqueues nothing.
 * Errors: ARG if n_blocks < 0 or n_blocks > capacity/4, a pointer is null or
 * q_idx is not 16-byte aligned. */
qsa_status qsa_index_score(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                           int32_t n_blocks, const float *q_idx, const float *w,
                           float *scores, hipStream_t stream);

/* Stage 3 [post 10, "QSA indexer"; "block-domain top-k（COMMON-006）実装は
 * 見送り"]: writes the min(k_blocks, n_blocks) ids ranked first by (score
 * descending, id ascending) to sel (DEVICE int32), in ascending id order.
 * -0.0 and +0.0 are equal; scores must be finite.  The result does not depend
 * on scheduling or atomic order.  scores: DEVICE fp32 [n_blocks].
 * Workspace >= qsa_workspace_bytes of any descriptor whose capacity >=
 * 4 * n_blocks.
 * Errors: ARG if n_blocks < 0, k_blocks < 1 or a pointer is null;
 * WORKSPACE if ws is null, misaligned or smaller than needed. */
qsa_status qsa_topk_blocks(const float *scores, int32_t n_blocks, int32_t k_blocks,
                           int32_t *sel, void *ws, size_t ws_bytes, hipStream_t stream);

/* Stage 4 [post 10, "selected QSA K/V gather（COMMON-005）"]: attention of
 * the current query over the cells {4*sel[i] + j : i < n_sel_blocks, j < 4}
 * followed by the tail cells 4*floor(n_tokens/4) .. n_tokens-1, reading only
 * those K/V rows.  sel: DEVICE int32 [n_sel_blocks], ascending, each id <
 * floor(n_tokens/4); may be NULL only when n_sel_blocks == floor(n_tokens/4)
 * (every block kept).  q: DEVICE fp32 [Hq][Dh]; out: DEVICE fp32 [Hq][Dh].
 * Split-context flash-decode: partial softmax states go to the workspace and
 * are merged in a fixed order, so results are bitwise repeatable.
 * Errors: ARG if n_tokens < 1, n_tokens > capacity, n_sel_blocks outside
 * [0, min(top_k_tokens/4, floor(n_tokens/4))], no cell to attend
 * (n_sel_blocks = 0 and n_tokens a multiple of 4) or a pointer is null;
 * WORKSPACE as above. */
qsa_status qsa_gather_attend(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                             int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                             const float *q, float *out, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* The fused decode step (stages 1-4 on one stream, no host synchronisation)
 * [post 10, all sections above].  Appends the new token at pos =
 * st->n_tokens: copies idx_k_row (DEVICE [H_i][D_i] idx_dtype), k_row and
 * v_row (DEVICE [Hkv][Dh] binary16) into the cache at row pos; n = pos + 1;
 * rebuilds summary rows [st->n_valid_blocks, n/4); scores, selects and
 * attends as above.  gamma, q_idx, w, q, out as in the stage calls.
 * sel_out (DEVICE int32 [min(K, n/4)]) and scores_out (DEVICE fp32 [n/4])
 * are optional (NULL to skip).  On success st becomes {n, n/4}; on any
 * error st is unchanged.
 * Errors: ARG if st->n_tokens < 0, pos >= capacity or a pointer is null;
 * UNSUPPORTED / WORKSPACE as above. */
qsa_status qsa_decode_step(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                           qsa_seq_state *st, const void *idx_k_row, const uint16_t *k_row,
                           const uint16_t *v_row, const float *gamma, const float *q_idx,
                           const float *w, const float *q, float *out, int32_t *sel_out,
                           float *scores_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- batches
 * Batched variable-length decode: one decode step (as qsa_decode_step) for
 * each of n_seq independent sequences of the same layer shapes, in one call:
 * one launch per stage for the whole batch, so short contexts share the GPU
 * instead of each filling it alone [post 10, "QSA indexer", "selected QSA K/V
 * gather（COMMON-005）": the same per-sequence step; batching is this
 * library's].  Sequence s has its own cache caches[s], state states[s] and
 * I/O io[s]; gamma is the layer's, shared.  Results are those of n_seq
 * qsa_decode_step calls. */
#define QSA_MAX_BATCH 8

typedef struct qsa_seq_io {
    const void *idx_k_row;      /* DEVICE [H_i][D_i] idx_dtype: the appended token's raw key */
    const uint16_t *k_row;      /* DEVICE [Hkv][Dh] binary16 */
    const uint16_t *v_row;      /* DEVICE [Hkv][Dh] binary16 */
    const float *q_idx;         /* DEVICE fp32 [H_i][D_i], 16-byte aligned */
    const float *w;             /* DEVICE fp32 [H_i] */
    const float *q;             /* DEVICE fp32 [Hq][Dh], 16-byte aligned */
    float *out;                 /* DEVICE fp32 [Hq][Dh] */
    int32_t *sel_out;           /* optional DEVICE int32 [min(K, n/4)] (NULL to skip) */
    float *scores_out;          /* optional DEVICE fp32 [n/4]: the fp32 score of every block,
                                   the values the top-k ranks (NULL to skip) */
} qsa_seq_io;

/* Workspace bytes for qsa_decode_step_batch over sequences of the given
 * capacities (tokens each); 0 if the desc, n_seq (1..QSA_MAX_BATCH) or a
 * capacity is invalid. */
size_t qsa_batch_workspace_bytes(const qsa_layer_desc *desc, int32_t n_seq,
                                 const int32_t *capacities);

/* One decode step of each of n_seq sequences (HOST arrays of n_seq entries:
 * caches, states, io).  Each sequence follows qsa_decode_step: it appends at
 * pos = states[s].n_tokens and on success states[s] becomes {n, n/4}; on any
 * error no state changes.
 * Errors: ARG if n_seq is outside [1, QSA_MAX_BATCH], an array or pointer is
 * null, a position is outside its cache or a pointer is misaligned;
 * UNSUPPORTED / WORKSPACE as in qsa_decode_step. */
qsa_status qsa_decode_step_batch(const qsa_layer_desc *desc, int32_t n_seq,
                                 const qsa_layer_cache *caches, qsa_seq_state *states,
                                 const qsa_seq_io *io, const float *gamma, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------- prefill chunk
 * n_q consecutive tokens of one sequence in one call, with the results of n_q
 * qsa_decode_step calls in a row [post 10, "QSA indexer", "incremental
 * pooled-key cache（COMMON-004）", "selected QSA K/V gather（COMMON-005）": the
 * per-token step; running a ubatch of tokens through it at once is this
 * library's].  Token i (0 <= i < n_q) is appended at pos_i = st->n_tokens + i;
 * its query sees n_i = pos_i + 1 tokens: the floor(n_i / 4) blocks completed
 * by then (a causal block mask -- never a block completed by a later token of
 * the chunk), of which it keeps the top K = top_k_tokens / 4 by its own
 * indexer score, plus its own tail of n_i mod 4 cells.  Every block the chunk
 * completes (and any below the watermark) is pooled first, in one launch.
 * Scoring runs as one f16 matrix-core GEMM of all queries against all blocks:
 * the query q_idx[i][h] * w[i][h] is scaled by a power of two and split into
 * two f16 halves so that the products keep fp32 accuracy (fp32 summaries are
 * split likewise).  A chunk of at most QSA_MAX_MULTI tokens runs as
 * qsa_decode_step_multi instead (same results; scores_out then written
 * whenever nb_last > 0).
 *
 * idx_k_rows: DEVICE [n_q][H_i][D_i] idx_dtype; k_rows, v_rows: DEVICE
 * [n_q][Hkv][Dh] binary16; q_idx: DEVICE fp32 [n_q][H_i][D_i]; w: DEVICE fp32
 * [n_q][H_i]; q: DEVICE fp32 [n_q][Hq][Dh]; out: DEVICE fp32 [n_q][Hq][Dh].
 * Rows, q_idx, q and out 16-byte aligned.  sel_out (optional, DEVICE int32
 * [n_q][K]): row i gets the min(K, floor(n_i/4)) chosen ids ascending, then
 * -1.  scores_out (optional, DEVICE fp32 [n_q][nb_last], nb_last =
 * floor((pos_0 + n_q) / 4)): written only when some query has more than K
 * blocks; entry (i, b) is query i's score of block b for b < floor(n_i / 4),
 * -INFINITY past it.
 * On success st becomes {pos_0 + n_q, nb_last}; on a failed argument check
 * nothing is enqueued, and on any error st is unchanged (after QSA_ERR_HIP
 * the kernels enqueued before the failing launch, the append of the chunk's
 * rows first, stay enqueued).
 * Errors: ARG if n_q is outside [1, QSA_MAX_CHUNK], a pointer is null or
 * misaligned, or pos_0 + n_q > capacity; UNSUPPORTED / WORKSPACE as in
 * qsa_decode_step (workspace >= qsa_chunk_workspace_bytes). */
#define QSA_MAX_CHUNK 4096

/* Workspace bytes for qsa_chunk_step of up to n_q tokens on a cache of the
 * given capacity; 0 if the desc, capacity or n_q is invalid. */
size_t qsa_chunk_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity, int32_t n_q);

qsa_status qsa_chunk_step(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                          qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                          const uint16_t *k_rows, const uint16_t *v_rows, const float *gamma,
                          const float *q_idx, const float *w, const float *q, float *out,
                          int32_t *sel_out, float *scores_out, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* qsa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its workspace is a static device array
 * of QSA_STATIC_SCRATCH_BYTES per GPU, part of the library's image: every
 * GPU the library runs on holds it until the process ends, and the call
 * allocates nothing.  Arguments, results and errors are those of
 * qsa_decode_step, plus QSA_ERR_WORKSPACE when the cache's workspace
 * (qsa_workspace_bytes(desc, capacity)) exceeds the static one.  With the
 * 4 x 128 f16 indexer, 16 / 2 x 256 attention and top 2048 tokens every
 * capacity the library takes fits (6.3 MiB at 2^21 tokens); shapes with many
 * KV heads or a much larger top-k can exceed it.
 * Every call on one GPU shares that GPU's array and its contents carry from
 * call to call: calls that may overlap on one GPU (different streams not
 * ordered with each other) race and give wrong results.  Stream-ordered calls
 * need nothing cleared: the decode step checks its histogram region's tag,
 * so a region left by another layer or sequence only makes the next call
 * take the full top-k (same results). */
#define QSA_STATIC_SCRATCH_BYTES (16u << 20)
qsa_status qsa_decode_step_static(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                  qsa_seq_state *st, const void *idx_k_row, const uint16_t *k_row,
                                  const uint16_t *v_row, const float *gamma, const float *q_idx,
                                  const float *w, const float *q, float *out, int32_t *sel_out,
                                  float *scores_out, hipStream_t stream);

/* Stage 2 of qsa_decode_step on its own [post 10, "QSA indexer": block scores
 * s_b = sum_h w_h <q_idx_h, summary_b,h>], as the step launches it: the score
 * pass over the floor(st->n_tokens / 4) completed blocks (no append, no
 * pooling, st is not changed), writing into the workspace the selection keys,
 * the per-tile candidate lists and the score histogram whenever there are
 * more than K = top_k_tokens / 4 blocks -- the same kernel, grid and outputs
 * as inside the step.  For timing or inspecting the step's dominant kernel.
 * It leaves the workspace's histogram region filled: the next
 * qsa_decode_step on that workspace finds it unclean and takes the full
 * top-k once (same results).
 * gamma: DEVICE fp32 [D_i]; q_idx: DEVICE fp32 [H_i][D_i] (16-byte aligned);
 * w: DEVICE fp32 [H_i]; scores_out (optional): DEVICE fp32 [n_tokens / 4].
 * Workspace >= qsa_workspace_bytes(desc, capacity).  With no block, or at
 * most K blocks and no scores_out, nothing is enqueued.
 * Errors: ARG if a pointer is null or misaligned or n_tokens is outside
 * [0, capacity]; UNSUPPORTED / WORKSPACE as in qsa_decode_step. */
qsa_status qsa_decode_score(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                            const qsa_seq_state *st, const float *gamma, const float *q_idx,
                            const float *w, float *scores_out, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* qsa_chunk_step with grouped-union attention [post 10 names a "QSA
 * grouped-union" that sped up prefill (opening paragraphs; "Vulkan版の
 * プロファイリングでTGが遅くなった原因を調べる"; "COMMON-004実装結果", the
 * prefill paragraph) and does not define it; this is a reading].
 * Consecutive queries of the chunk form groups of min(64 / G, 32) (G =
 * q_heads / kv_heads: 64 query x head rows, four matrix-core tiles; fewer
 * when the group's bitmaps of ceil(n_blocks / 32) words per query would
 * exceed 128 KB); a group reads the K / V rows of the union of its queries'
 * chosen blocks and of its queries' tail cells once, and each query attends
 * over that union with the cells that are not its own masked out.  Results,
 * arguments, workspace (qsa_chunk_workspace_bytes covers both) and errors
 * are qsa_chunk_step's, plus UNSUPPORTED when no group fits; outputs equal
 * qsa_chunk_step's up to the order of the softmax sums.  A chunk of at most
 * QSA_MAX_MULTI tokens runs as qsa_decode_step_multi, as there. */
qsa_status qsa_chunk_step_grouped(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                  qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                                  const uint16_t *k_rows, const uint16_t *v_rows, const float *gamma,
                                  const float *q_idx, const float *w, const float *q, float *out,
                                  int32_t *sel_out, float *scores_out, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------ multi-query decode
 * Speculative verification: the token at pos_0 = st->n_tokens and up to
 * QSA_MAX_MULTI - 1 drafted tokens after it, decoded in one call with the
 * results of n_q qsa_decode_step calls in a row [post 10, "QSA indexer",
 * "incremental pooled-key cache（COMMON-004）", "selected QSA K/V gather
 * （COMMON-005）": the per-token step; running a few tokens of one sequence
 * through it together is this library's].  Token i is appended at pos_i =
 * pos_0 + i and its query sees n_i = pos_i + 1 tokens: the floor(n_i / 4)
 * blocks completed by then (never a block completed by a later token of the
 * call), its own top K = top_k_tokens / 4 of them by its own indexer score,
 * and its tail of n_i mod 4 cells.  Every summary row is read once for all
 * queries; the top-k and the gather-attention run per query.
 *
 * Rejected drafts [dirty-range protection; post 10, COMMON-004 section: the
 * cache is invalidated on a sequence edit]: after accepting a tokens of the
 * call, qsa_state_truncate(st, pos_0 + a) drops the rest and lowers the
 * summary watermark below any block that held a dropped token, so the next
 * step that completes that block pools it again from the rows then in the
 * cache.  Rows of dropped tokens are overwritten by the next appends.
 *
 * Arguments and layouts as in qsa_chunk_step (idx_k_rows [n_q][H_i][D_i],
 * k_rows / v_rows [n_q][Hkv][Dh], q_idx [n_q][H_i][D_i], w [n_q][H_i], q and
 * out [n_q][Hq][Dh], all DEVICE, rows, q_idx, q and out 16-byte aligned).
 * sel_out (optional, DEVICE int32 [n_q][K]): row i gets the min(K,
 * floor(n_i/4)) chosen ids ascending, then -1.  scores_out (optional, DEVICE
 * fp32 [n_q][nb_last], nb_last = floor((pos_0 + n_q) / 4)): entry (i, b) is
 * query i's score of block b for b < floor(n_i / 4), -INFINITY past it
 * (written whenever nb_last > 0).  Workspace >= qsa_multi_workspace_bytes.
 * On success st becomes {pos_0 + n_q, nb_last}; on a failed argument check
 * nothing is enqueued, and on any error st is unchanged (after QSA_ERR_HIP
 * the kernels enqueued before the failing launch, the append of the call's
 * rows first, stay enqueued).
 * Errors: ARG if n_q is outside [1, QSA_MAX_MULTI], a pointer is null or
 * misaligned, or pos_0 + n_q > capacity; UNSUPPORTED / WORKSPACE as in
 * qsa_decode_step. */
#define QSA_MAX_MULTI 4

/* Workspace bytes for qsa_decode_step_multi of up to n_q tokens on a cache of
 * the given capacity; 0 if the desc, capacity or n_q is invalid. */
size_t qsa_multi_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity, int32_t n_q);

qsa_status qsa_decode_step_multi(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                                 qsa_seq_state *st, int32_t n_q, const void *idx_k_rows,
                                 const uint16_t *k_rows, const uint16_t *v_rows,
                                 const float *gamma, const float *q_idx, const float *w,
                                 const float *q, float *out, int32_t *sel_out, float *scores_out,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ ablations
 * The page's comparisons of its own changes, reproduced as library calls so
 * that each can be timed on this hardware against the path above.  (The
 * third, the pooled-key cache switched off, needs no call of its own:
 * qsa_state_invalidate(st, 0) before a qsa_decode_step pools every block
 * again.) */

/* Workspace bytes for qsa_topk_cells and qsa_attend_masked on a cache of the
 * given capacity; 0 for an invalid descriptor or capacity. */
size_t qsa_ablation_workspace_bytes(const qsa_layer_desc *desc, int32_t capacity);

/* The selection as the page made it before its block-domain top-k [post 10,
 * "block-domain top-k（COMMON-006）実装は見送り": block scores copied to every
 * cell of the block, then a top-k over the cells]: cell 4b + j gets s[b];
 * the top_k_tokens cells ranked first by (score descending, cell
 * ascending), in ascending order, then the tail cells 4 floor(n/4) .. n-1.
 * Because the 4 cells of a block tie and are consecutive, these are the
 * cells of the blocks qsa_topk_blocks chooses with k = top_k_tokens / 4.
 * block_scores: DEVICE fp32 [floor(n_tokens/4)]; cells: DEVICE int32
 * [min(top_k_tokens, 4 floor(n/4)) + n mod 4].  Workspace >=
 * qsa_ablation_workspace_bytes of any descriptor whose capacity >= n_tokens.
 * Errors: ARG if n_tokens < 1, floor(n_tokens/4) > 2^17, top_k_tokens is
 * not a positive multiple of 4 or a pointer is null; WORKSPACE as in
 * qsa_topk_blocks. */
qsa_status qsa_topk_cells(const float *block_scores, int32_t n_tokens, int32_t top_k_tokens,
                          int32_t *cells, void *ws, size_t ws_bytes, hipStream_t stream);

/* The attention with the gather switched off [post 10, "selected QSA K/V
 * gather（COMMON-005）": before it, flash attention ran over the whole cache
 * with the unselected cells masked]: reads every cached K / V row of the n
 * tokens; cells of blocks outside sel get no weight, the tail cells always
 * take part.  The result is that of qsa_gather_attend with the same
 * arguments (up to summation order).  sel: DEVICE int32 [n_sel_blocks],
 * ascending, each < floor(n_tokens/4); q, out: DEVICE fp32 [Hq][Dh],
 * 16-byte aligned.  Workspace >= qsa_ablation_workspace_bytes.
 * Errors: ARG if n_tokens is outside [1, capacity], n_sel_blocks outside
 * [0, floor(n_tokens/4)], no cell to attend (n_sel_blocks = 0 and n_tokens a
 * multiple of 4), sel is null with n_sel_blocks > 0, or q / out is null or
 * misaligned; UNSUPPORTED / WORKSPACE as in qsa_gather_attend. */
qsa_status qsa_attend_masked(const qsa_layer_desc *desc, const qsa_layer_cache *cache,
                             int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                             const float *q, float *out, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------ q8_0 K/V
 * The 8-bit K/V cache type the runtime-tuning post tried (section "KV
 * cacheをQ8_0にしてみる": llama.cpp's q8_0; the post saw no speed gain on its
 * APU and names no layout).  q8_0 is llama.cpp's published format: each 32
 * consecutive values of a row share one binary16 scale d = amax / 127 and
 * are stored as int8 codes round(x / d), halves away from zero; value =
 * code * d.  Here the codes and the scales live in two planes (the values
 * are those of the format; only the layout differs from llama.cpp's
 * interleaved 34-byte blocks, so that code loads stay aligned):
 *   codes  [capacity][Hkv][Dh] int8, row t = position t;
 *   scales [capacity][Hkv][Dh/32] binary16 bits.
 * The library quantises (qsa_q8_0_quantize) and attends
 * (qsa_gather_attend_q8_0); the caller owns the planes.  Scoring, top-k and
 * the pooled-key cache are unchanged (they never read K/V). */
typedef struct {
    const int8_t *k_codes;     /* DEVICE [capacity][Hkv][Dh], 16-byte aligned */
    const uint16_t *k_scales;  /* DEVICE [capacity][Hkv][Dh/32] binary16, 16-byte aligned */
    const int8_t *v_codes;
    const uint16_t *v_scales;
    int32_t capacity;          /* tokens; a positive multiple of 4, <= 2^21 */
} qsa_kv_q8_0;

/* q8_0 of n_values binary16 values (n_values a multiple of 32; blocks of 32
 * consecutive values).  The decisions are taken in binary32 (correctly
 * rounded amax / 127, its reciprocal and the product), the scale stored
 * rounded to nearest-even binary16.  To quantise cache rows [t0, t1) pass
 * x = the f16 rows, codes = k_codes + t0 * Hkv * Dh, scales = k_scales +
 * t0 * Hkv * Dh / 32 and n_values = (t1 - t0) * Hkv * Dh.  x: DEVICE, 16-byte
 * aligned; codes: DEVICE, 16-byte aligned; scales: DEVICE, 2-byte aligned.
 * Inputs must be finite.  n_values = 0 enqueues nothing.
 * Errors: ARG if n_values < 0 or not a multiple of 32, or a pointer is null
 * or misaligned. */
qsa_status qsa_q8_0_quantize(const uint16_t *x, int64_t n_values, int8_t *codes, uint16_t *scales,
                             hipStream_t stream);

/* Stage 4 over a q8_0 K/V cache: the attention of qsa_gather_attend
 * [post 10, "selected QSA K/V gather（COMMON-005）"] with every K and V
 * element read as code * scale: the same cells (sel blocks + tail), softmax
 * over scale * <q_h, K_c>, weighted sum of V.  Reads n_sel * Hkv * (Dh + Dh/16)
 * bytes per K and per V, about half of the f16 gather.  Arguments as in
 * qsa_gather_attend, with kv in place of the cache; q and out 16-byte
 * aligned; workspace >= qsa_workspace_bytes(desc, kv->capacity).
 * Errors: ARG as in qsa_gather_attend (and a null or misaligned kv pointer,
 * q or out); UNSUPPORTED / WORKSPACE as there. */
qsa_status qsa_gather_attend_q8_0(const qsa_layer_desc *desc, const qsa_kv_q8_0 *kv,
                                  int32_t n_tokens, const int32_t *sel, int32_t n_sel_blocks,
                                  const float *q, float *out, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Static text for a status code. */
const char *qsa_status_string(qsa_status s);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" if none). */
const char *qsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H */
