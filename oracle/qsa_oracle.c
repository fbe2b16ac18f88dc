/*
 * qsa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU model of one QSA (Qwen Sparse
 * Attention) decode step, written in scalar C with every intermediate in
 * IEEE double.  Only the test suite, the smoke entry point and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the GPU library; it is never a fallback for it.
 *
 * Source pages (public blog posts by "ariera" on qiita.com):
 *   [post 10] "第10回 EVO-X2（Ryzen AI Max+ 395 / 128GB）+ Qwen3.8-Flash-Next用の
 *              llama.cpp改造で長コンテキストのTGを高速化した話"
 * Sections are cited by their headings, e.g. [post 10, "QSA indexer"].
 *
 * What the pages fix, restated:
 *   - indexer keys are grouped into 4-token micro-blocks; each block is
 *     average-pooled, RMS-normalised, then rotated by RoPE, giving one
 *     summary row per block; the query is scored against the summaries and
 *     the highest-scoring blocks are kept [post 10, "QSA indexer"];
 *   - top-k is 2048 tokens with compression 4, so at most 2048 + 4 - 1 cells
 *     reach attention, counting the unfinished current block
 *     [post 10, "QSA indexer"; "なぜFlash Attentionがcontext長に比例していたのか"];
 *   - summaries of completed blocks are cached per layer and only new or
 *     invalidated blocks are recomputed [post 10, "incremental pooled-key
 *     cache（COMMON-004）"];
 *   - top-k is taken in the block domain and only the chosen blocks are
 *     expanded to cells, with the tail cells appended [post 10,
 *     "block-domain top-k（COMMON-006）実装は見送り"];
 *   - the chosen K/V rows are gathered and ordinary attention runs over them
 *     [post 10, "selected QSA K/V gather（COMMON-005）"].
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   R1 score = sum_h w_h * <q_h, khat_h>, no activation, no extra scale;
 *   R2 RMSNorm per head over D with eps inside the root, gamma[D] shared
 *      by all heads;
 *   R3 RoPE pairs element j with j + D/2 ("NeoX" half split), frequency
 *      theta^(-2j/D), position p = 4*b (block start), angle in double;
 *   R4 a summary is rounded once (round-to-nearest-even) to the storage type
 *      of the raw keys (f16 or f32) and scored as stored;
 *   R5 top-k orders by (score descending, block index ascending); -0 == +0;
 *      the chosen ids are returned ascending;
 *   R6 the tail (n mod 4 cells) is always attended and never scored;
 *   R7 attention scale 1/sqrt(Dh), contiguous GQA groups, no mask.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_F16 1

/* ---- storage conversions (IEEE binary16 / binary32) -------------------- */

double qsa_oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                    /* zero / subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25);      /* 1.man * 2^(ex-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t qsa_oracle_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return sign | 0x7e00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; 1024 quanta encodes the smallest normal */
        double r = nearbyint(a * 16777216.0);
        return sign | (uint16_t)r;
    }
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int E = e - 1;                      /* unbiased exponent */
    if (E > 15)
        return sign | 0x7c00;
    double r = nearbyint(ldexp(a, 10 - E));   /* significand * 1024, in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
        if (E > 15)
            return sign | 0x7c00;
    }
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024);
}

static double load_elem(const void *base, int dtype, size_t i)
{
    if (dtype == ORACLE_F16)
        return qsa_oracle_half_to_double(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

static void store_elem(void *base, int dtype, size_t i, double v)
{
    if (dtype == ORACLE_F16)
        ((uint16_t *)base)[i] = qsa_oracle_double_to_half(v);
    else
        ((float *)base)[i] = (float)v;       /* C cast: round to nearest even */
}

/* ---- O1..O3: one block summary in double --------------------------------
 * raw:   [tokens][H][D] raw indexer keys (dtype), row t = position t
 * out:   [H][D] summary of block b before storage rounding
 * Mean of the 4 rows of the block, RMS norm per head, then RoPE at the
 * block's start position [post 10, "QSA indexer"] (readings R2, R3).
 */
void qsa_oracle_summary_row(const void *raw, int dtype, int H, int D, long b,
                            const float *gamma, double eps, double theta,
                            double *out)
{
    const size_t row = (size_t)H * D;
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    const double p = 4.0 * (double)b;
    for (int h = 0; h < H; ++h) {
        /* O1: arithmetic mean of the 4 tokens of the block */
        for (int i = 0; i < D; ++i) {
            double s = 0.0;
            for (int j = 0; j < 4; ++j)
                s += load_elem(raw, dtype, (size_t)(4 * b + j) * row + (size_t)h * D + i);
            y[i] = s / 4.0;
        }
        /* O2: RMS normalisation over the head's D values, then gamma */
        double ms = 0.0;
        for (int i = 0; i < D; ++i)
            ms += y[i] * y[i];
        ms /= (double)D;
        const double r = sqrt(ms + eps);
        for (int i = 0; i < D; ++i)
            y[i] = y[i] / r * (double)gamma[i];
        /* O3: rotate pair (j, j + D/2) by p * theta^(-2j/D) */
        const int half = D / 2;
        for (int j = 0; j < half; ++j) {
            const double phi = p * pow(theta, -2.0 * (double)j / (double)D);
            const double c = cos(phi), s = sin(phi);
            out[(size_t)h * D + j] = y[j] * c - y[j + half] * s;
            out[(size_t)h * D + j + half] = y[j] * s + y[j + half] * c;
        }
    }
    free(y);
}

/* RoPE alone at an arbitrary position (used by the invariance pins). */
void qsa_oracle_rope(const double *x, int D, double pos, double theta, double *out)
{
    const int half = D / 2;
    for (int j = 0; j < half; ++j) {
        const double phi = pos * pow(theta, -2.0 * (double)j / (double)D);
        const double c = cos(phi), s = sin(phi);
        out[j] = x[j] * c - x[j + half] * s;
        out[j + half] = x[j] * s + x[j + half] * c;
    }
}

/* ---- O4 + O9: (re)build stored summary rows [b0, b1) ---------------------
 * summary: [blocks][H][D] in the raw-key dtype (reading R4).
 * Rows are independent, so the loop may run in parallel without changing
 * any result.
 */
void qsa_oracle_cache_update(const void *raw, void *summary, int dtype, int H, int D,
                             long b0, long b1, const float *gamma, double eps,
                             double theta)
{
    const size_t row = (size_t)H * D;
    long b;
#pragma omp parallel for schedule(static)
    for (b = b0; b < b1; ++b) {
        double *tmp = (double *)malloc(sizeof(double) * row);
        qsa_oracle_summary_row(raw, dtype, H, D, b, gamma, eps, theta, tmp);
        for (size_t i = 0; i < row; ++i)
            store_elem(summary, dtype, (size_t)b * row + i, tmp[i]);
        free(tmp);
    }
}

/* ---- O5: indexer score of every stored block -----------------------------
 * s[b] = sum_h w[h] * sum_i q[h][i] * khat[b][h][i]  (reading R1)
 * a[b] = sum_h |w[h]| * sum_i |q[h][i] * khat[b][h][i]|, the scale of the
 *        rounding error of any evaluation order (nullable).
 * [post 10, "QSA indexer"]
 */
void qsa_oracle_scores(const void *summary, int dtype, long nb, int H, int D,
                       const float *q, const float *w, double *s, double *a)
{
    const size_t row = (size_t)H * D;
    long b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < nb; ++b) {
        double tot = 0.0, mag = 0.0;
        for (int h = 0; h < H; ++h) {
            double dot = 0.0, adot = 0.0;
            for (int i = 0; i < D; ++i) {
                const double t = (double)q[(size_t)h * D + i] *
                                 load_elem(summary, dtype, (size_t)b * row + (size_t)h * D + i);
                dot += t;
                adot += fabs(t);
            }
            tot += (double)w[h] * dot;
            mag += fabs((double)w[h]) * adot;
        }
        s[b] = tot;
        if (a)
            a[b] = mag;
    }
}

/* ---- O6: block-domain top-k ------------------------------------------------
 * Sort block ids by (score desc, id asc), keep the first min(k, nb), return
 * them ascending.  Comparison in double treats -0 and +0 as equal.
 * [post 10, "QSA indexer"; "block-domain top-k（COMMON-006）実装は見送り"]
 */
static const double *g_sort_scores;   /* qsort has no context argument */

static int cmp_rank(const void *x, const void *y)
{
    const int32_t i = *(const int32_t *)x, j = *(const int32_t *)y;
    const double si = g_sort_scores[i], sj = g_sort_scores[j];
    if (si > sj) return -1;
    if (si < sj) return 1;
    return (i > j) - (i < j);
}

static int cmp_id(const void *x, const void *y)
{
    const int32_t i = *(const int32_t *)x, j = *(const int32_t *)y;
    return (i > j) - (i < j);
}

long qsa_oracle_topk(const double *s, long nb, long k, int32_t *sel)
{
    if (nb <= 0 || k <= 0)
        return 0;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)nb);
    for (long b = 0; b < nb; ++b)
        ids[b] = (int32_t)b;
    g_sort_scores = s;
    qsort(ids, (size_t)nb, sizeof(int32_t), cmp_rank);
    const long kb = k < nb ? k : nb;
    memcpy(sel, ids, sizeof(int32_t) * (size_t)kb);
    qsort(sel, (size_t)kb, sizeof(int32_t), cmp_id);
    free(ids);
    return kb;
}

/* ---- O7: cells that reach attention -----------------------------------------
 * The 4 cells of every chosen block, then the tail cells 4*floor(n/4) .. n-1.
 * Returns the count 4*kb + (n mod 4).
 * [post 10, "なぜFlash Attentionがcontext長に比例していたのか"; COMMON-006 section]
 */
long qsa_oracle_cells(const int32_t *sel, long kb, long n, int32_t *cells)
{
    long c = 0;
    for (long i = 0; i < kb; ++i)
        for (int j = 0; j < 4; ++j)
            cells[c++] = 4 * sel[i] + j;
    for (long t = 4 * (n / 4); t < n; ++t)
        cells[c++] = (int32_t)t;
    return c;
}

/* ---- O8: attention over the gathered cells ---------------------------------
 * q:    [Hq][Dh] fp32;  K, V: [tokens][Hkv][Dh] f16 bits;  out: [Hq][Dh]
 * Head h uses KV head floor(h * Hkv / Hq); logits scale * <q_h, K_c>;
 * max-subtracted softmax over the listed cells; weighted sum of V rows.
 * [post 10, "selected QSA K/V gather（COMMON-005）"] (reading R7)
 */
void qsa_oracle_attend(const float *q, const uint16_t *K, const uint16_t *V,
                       const int32_t *cells, long nc, int Hq, int Hkv, int Dh,
                       double scale, double *out)
{
    const size_t row = (size_t)Hkv * Dh;
    int h;
    /* heads are independent: each thread runs the same per-head arithmetic */
#pragma omp parallel for schedule(static)
    for (h = 0; h < Hq; ++h) {
        double *lg = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
        const int g = (int)(((long)h * Hkv) / Hq);
        double mx = -INFINITY;
        for (long c = 0; c < nc; ++c) {
            const size_t base = (size_t)cells[c] * row + (size_t)g * Dh;
            double dot = 0.0;
            for (int d = 0; d < Dh; ++d)
                dot += (double)q[(size_t)h * Dh + d] * qsa_oracle_half_to_double(K[base + d]);
            lg[c] = scale * dot;
            if (lg[c] > mx)
                mx = lg[c];
        }
        double z = 0.0;
        for (long c = 0; c < nc; ++c) {
            lg[c] = exp(lg[c] - mx);
            z += lg[c];
        }
        for (int d = 0; d < Dh; ++d) {
            double acc = 0.0;
            for (long c = 0; c < nc; ++c)
                acc += lg[c] * qsa_oracle_half_to_double(V[(size_t)cells[c] * row + (size_t)g * Dh + d]);
            out[(size_t)h * Dh + d] = acc / z;
        }
        free(lg);
    }
}

/* ---- grouped-union prefill attention (a reading) --------------------------
 * Post 10 (opening paragraphs; "Vulkan版のプロファイリングでTGが遅くなった
 * 原因を調べる"; "COMMON-004実装結果", the prefill paragraph) names a "QSA
 * grouped-union" that sped up prefill in an earlier build and does not define
 * it.  Reading: consecutive queries of a prefill chunk form a group; the
 * group reads the K / V rows of the UNION of its queries' chosen blocks, and
 * of the cells from the first query's completed blocks to the last query's
 * token (the queries' tails), once, and each query attends over that union
 * with every cell outside its own cells masked out -- so each query's result
 * is its own QSA attention (chosen blocks' cells and its tail).
 *
 * qsa_oracle_union_blocks: the union of nq ascending id lists (query i's
 * ids at sel[i * kb .. + ksel[i])), ascending, into uni (capacity cap);
 * returns its size (or -1 past cap). */
static int cmp_i32(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

long qsa_oracle_union_blocks(const int32_t *sel, const int32_t *ksel, int nq, int kb, int32_t *uni, long cap)
{
    long m = 0;
    for (int i = 0; i < nq; ++i)
        m += ksel[i];
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
    long p = 0;
    for (int i = 0; i < nq; ++i)
        for (int j = 0; j < ksel[i]; ++j)
            all[p++] = sel[(size_t)i * kb + j];
    qsort(all, (size_t)m, sizeof(int32_t), cmp_i32);
    long u = 0;
    for (long j = 0; j < m; ++j) {
        if (j > 0 && all[j] == all[j - 1])
            continue;
        if (u >= cap) {
            free(all);
            return -1;
        }
        uni[u++] = all[j];
    }
    free(all);
    return u;
}

/* Whether id is in the ascending list l[0 .. len). */
static int in_sorted(const int32_t *l, int len, int32_t id)
{
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (l[mid] < id)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo < len && l[lo] == id;
}

/* qsa_oracle_union_attend: q [nq][Hq][Dh] fp32; n[i] tokens seen by query i;
 * sel / ksel / kb as above (each query's ids below n[i] / 4); K, V
 * [tokens][Hkv][Dh] binary16; out [nq][Hq][Dh].  Steps: the union of the
 * ids; its cells (4 per block, ascending) followed by the group's tail range
 * [4 floor(n_first / 4), n_last); for each query and head a softmax over
 * those cells with a cell counting only when it is one of the query's own
 * (in one of its chosen blocks, or in [4 floor(n_i / 4), n_i)). */
void qsa_oracle_union_attend(const float *q, const uint16_t *K, const uint16_t *V, const int32_t *sel,
                             const int32_t *ksel, const int64_t *n, int nq, int kb, int Hq, int Hkv, int Dh,
                             double scale, double *out)
{
    long cap = (long)nq * kb + 1;
    int32_t *uni = (int32_t *)malloc(sizeof(int32_t) * (size_t)cap);
    const long nu = qsa_oracle_union_blocks(sel, ksel, nq, kb, uni, cap);
    int64_t t0 = n[0] / 4 * 4, t1 = n[0];
    for (int i = 1; i < nq; ++i) {
        if (n[i] / 4 * 4 < t0)
            t0 = n[i] / 4 * 4;
        if (n[i] > t1)
            t1 = n[i];
    }
    const long ncell = 4 * nu + (long)(t1 - t0);
    int64_t *cell = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ncell > 0 ? ncell : 1));
    for (long u = 0; u < nu; ++u)
        for (int r = 0; r < 4; ++r)
            cell[4 * u + r] = 4 * (int64_t)uni[u] + r;
    for (int64_t c = t0; c < t1; ++c)
        cell[4 * nu + (c - t0)] = c;
    const size_t row = (size_t)Hkv * Dh;
    double *lg = (double *)malloc(sizeof(double) * (size_t)(ncell > 0 ? ncell : 1));
    char *own = (char *)malloc((size_t)(ncell > 0 ? ncell : 1));
    for (int i = 0; i < nq; ++i) {
        const int32_t *si = sel + (size_t)i * kb;
        const int64_t tail0 = n[i] / 4 * 4;
        for (long c = 0; c < ncell; ++c) {
            if (c < 4 * nu)
                own[c] = (char)in_sorted(si, ksel[i], uni[c / 4]);
            else
                own[c] = (char)(cell[c] >= tail0 && cell[c] < n[i]);
        }
        for (int h = 0; h < Hq; ++h) {
            const int g = (int)(((long)h * Hkv) / Hq);
            const float *qh = q + ((size_t)i * Hq + h) * Dh;
            double mx = -INFINITY;
            for (long c = 0; c < ncell; ++c) {
                if (!own[c])
                    continue;
                const size_t base = (size_t)cell[c] * row + (size_t)g * Dh;
                double dot = 0.0;
                for (int d = 0; d < Dh; ++d)
                    dot += (double)qh[d] * qsa_oracle_half_to_double(K[base + d]);
                lg[c] = scale * dot;
                if (lg[c] > mx)
                    mx = lg[c];
            }
            double z = 0.0;
            for (long c = 0; c < ncell; ++c) {
                lg[c] = own[c] ? exp(lg[c] - mx) : 0.0;
                z += lg[c];
            }
            for (int d = 0; d < Dh; ++d) {
                double acc = 0.0;
                for (long c = 0; c < ncell; ++c)
                    if (own[c])
                        acc += lg[c] * qsa_oracle_half_to_double(V[(size_t)cell[c] * row + (size_t)g * Dh + d]);
                out[((size_t)i * Hq + h) * Dh + d] = acc / z;
            }
        }
    }
    free(own);
    free(lg);
    free(cell);
    free(uni);
}

/* ---- q8_0 K/V: 8-bit codes, one binary16 scale per 32 values --------------
 * The tuning post (the one on runtime parameters, section "KV cacheをQ8_0に
 * してみる") runs llama.cpp with its q8_0 K/V cache type and gives no format;
 * q8_0 is llama.cpp's published one: 32 consecutive values share a scale.
 * Reading, in the format's own precision (binary32 decisions):
 *   amax = max_j |x_j|;  s = amax / 127;  inv = (s != 0) ? 1 / s : 0;
 *   code_j = round(x_j * inv), halves away from zero (|code_j| <= 127);
 *   the scale is stored as s rounded to nearest-even binary16 (d16), and
 *   value j is code_j * d16.
 * x: n_blocks * 32 binary16 values; codes: as many int8; d: n_blocks scales.
 */
void qsa_oracle_q8_0_quantize(const uint16_t *x, long n_blocks, int8_t *codes, uint16_t *d)
{
    for (long b = 0; b < n_blocks; ++b) {
        float v[32];
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            v[j] = (float)qsa_oracle_half_to_double(x[b * 32 + j]);
            if (fabsf(v[j]) > amax)
                amax = fabsf(v[j]);
        }
        const float s = amax / 127.0f;
        const float inv = s != 0.0f ? 1.0f / s : 0.0f;
        for (int j = 0; j < 32; ++j) {
            const float t = v[j] * inv;
            codes[b * 32 + j] = (int8_t)roundf(t);
        }
        d[b] = qsa_oracle_double_to_half((double)s);
    }
}

/* Value i of a q8_0 tensor (blocks of 32 consecutive values). */
static double q8_value(const int8_t *codes, const uint16_t *d, size_t i)
{
    return (double)codes[i] * qsa_oracle_half_to_double(d[i / 32]);
}

/* O8 over a q8_0 K/V cache: the same attention as qsa_oracle_attend, with
 * every K and V element read as code * scale.  Kc/Vc: [tokens][Hkv][Dh]
 * codes; Kd/Vd: [tokens][Hkv][Dh/32] scales (Dh a multiple of 32). */
void qsa_oracle_attend_q8_0(const float *q, const int8_t *Kc, const uint16_t *Kd,
                            const int8_t *Vc, const uint16_t *Vd, const int32_t *cells, long nc,
                            int Hq, int Hkv, int Dh, double scale, double *out)
{
    double *lg = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
    const size_t row = (size_t)Hkv * Dh;
    for (int h = 0; h < Hq; ++h) {
        const int g = (int)(((long)h * Hkv) / Hq);
        double mx = -INFINITY;
        for (long c = 0; c < nc; ++c) {
            const size_t base = (size_t)cells[c] * row + (size_t)g * Dh;
            double dot = 0.0;
            for (int e = 0; e < Dh; ++e)
                dot += (double)q[(size_t)h * Dh + e] * q8_value(Kc, Kd, base + e);
            lg[c] = scale * dot;
            if (lg[c] > mx)
                mx = lg[c];
        }
        double z = 0.0;
        for (long c = 0; c < nc; ++c) {
            lg[c] = exp(lg[c] - mx);
            z += lg[c];
        }
        for (int e = 0; e < Dh; ++e) {
            double acc = 0.0;
            for (long c = 0; c < nc; ++c)
                acc += lg[c] * q8_value(Vc, Vd, (size_t)cells[c] * row + (size_t)g * Dh + e);
            out[(size_t)h * Dh + e] = acc / z;
        }
    }
    free(lg);
}

/* Harness helpers (no arithmetic of the method): the OpenMP threads the
 * parallel loops above use, and a way to set them (1 = the serial oracle). */
int qsa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void qsa_oracle_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
