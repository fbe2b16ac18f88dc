// qsa_pool.h -- device code of stage 1 (append + pool one summary row), shared
// by the stand-alone update kernel and the score kernel's fused prologue.
//
// Row layout: wave h of a 256-thread workgroup owns indexer head h; lane j owns
// the RoPE pair (j, j + D/2), so the rotation needs no exchange and the RMS norm
// is one wave reduction.  Mean, mean-square, normalisation and rotation run in
// double: the angle 4b * theta^(-2j/D) reaches ~2.6e5 rad at 256k context,
// where a float angle is off by up to ~1e-2 rad.  The result is rounded once
// (to nearest even) to the storage dtype.
// [post 10, "QSA indexer"; "incremental pooled-key cache（COMMON-004）"]
#pragma once
#include "qsa_internal.h"

namespace qsa {

// Round a double to binary16, ties to even, directly (a float detour could
// round twice).
__device__ inline uint16_t f64_to_f16_rne(double x)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a >= 0x7FF0000000000000ull)
        return sign | (a > 0x7FF0000000000000ull ? 0x7E00 : 0x7C00);
    const int e = (int)(a >> 52) - 1023;
    if (e > 15)
        return sign | 0x7C00;
    const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    const int shift = e >= -14 ? 42 : 42 + (-14 - e);   // bits below the binary16 quantum
    if (shift > 63)
        return sign;
    const uint64_t keep = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t halfq = 1ull << (shift - 1);
    const uint64_t q = keep + ((rem > halfq || (rem == halfq && (keep & 1))) ? 1 : 0);
    if (e >= -14)   // a carry out of the significand bumps the exponent field
        return sign | (uint16_t)(((uint32_t)(e + 15) << 10) + (uint32_t)(q - 1024));
    return sign | (uint16_t)q;   // subnormal; q == 1024 encodes the smallest normal
}

template <bool F16>
__device__ inline double load_idx(const void *p, size_t i)
{
    if constexpr (F16)
        return (double)((const _Float16 *)p)[i];
    else
        return (double)((const float *)p)[i];
}

// Copy the n_new appended tokens' raw indexer-key, K and V rows (consecutive
// in their sources) into the caches (threads of one workgroup, any count).
__device__ inline void append_rows(const UpdateArgs &a, int t, int nthreads)
{
    const uint32_t *src = (const uint32_t *)a.new_idx_row;
    uint32_t *dst = (uint32_t *)a.idx_k + (size_t)a.pos * a.idx_row_words;
    const int iw = a.n_new * a.idx_row_words;
    for (int i = t; i < iw; i += nthreads)
        dst[i] = src[i];
    const uint32_t *sk = (const uint32_t *)a.new_k_row;
    const uint32_t *sv = (const uint32_t *)a.new_v_row;
    uint32_t *dk = (uint32_t *)a.k + (size_t)a.pos * a.kv_row_words;
    uint32_t *dv = (uint32_t *)a.v + (size_t)a.pos * a.kv_row_words;
    const int kw = a.n_new * a.kv_row_words;
    for (int i = t; i < kw; i += nthreads) {
        dk[i] = sk[i];
        dv[i] = sv[i];
    }
}

// The append split in two for a caller that streams other rows meanwhile:
// append_fetch loads the first kAppendPre words per thread of each appended
// row into registers, append_put stores them and copies whatever lies past
// them word by word.  Together they do what append_rows does.
constexpr int kAppendPre = 2;

struct AppendWords {
    uint32_t idx[kAppendPre], k[kAppendPre], v[kAppendPre];
};

__device__ inline void append_fetch(const UpdateArgs &a, int t, int nthreads, AppendWords &w)
{
    const uint32_t *src = (const uint32_t *)a.new_idx_row;
    const uint32_t *sk = (const uint32_t *)a.new_k_row;
    const uint32_t *sv = (const uint32_t *)a.new_v_row;
    const int iw = a.n_new * a.idx_row_words;
    const int kw = a.n_new * a.kv_row_words;
#pragma unroll
    for (int m = 0; m < kAppendPre; ++m) {
        const int i = t + nthreads * m;
        w.idx[m] = i < iw ? src[i] : 0u;
        w.k[m] = i < kw ? sk[i] : 0u;
        w.v[m] = i < kw ? sv[i] : 0u;
    }
}

__device__ inline void append_put(const UpdateArgs &a, int t, int nthreads, const AppendWords &w)
{
    const uint32_t *src = (const uint32_t *)a.new_idx_row;
    uint32_t *dst = (uint32_t *)a.idx_k + (size_t)a.pos * a.idx_row_words;
    const uint32_t *sk = (const uint32_t *)a.new_k_row;
    const uint32_t *sv = (const uint32_t *)a.new_v_row;
    uint32_t *dk = (uint32_t *)a.k + (size_t)a.pos * a.kv_row_words;
    uint32_t *dv = (uint32_t *)a.v + (size_t)a.pos * a.kv_row_words;
    const int iw = a.n_new * a.idx_row_words;
    const int kw = a.n_new * a.kv_row_words;
#pragma unroll
    for (int m = 0; m < kAppendPre; ++m) {
        const int i = t + nthreads * m;
        if (i < iw)
            dst[i] = w.idx[m];
        if (i < kw) {
            dk[i] = w.k[m];
            dv[i] = w.v[m];
        }
    }
    for (int i = t + nthreads * kAppendPre; i < iw; i += nthreads)
        dst[i] = src[i];
    for (int i = t + nthreads * kAppendPre; i < kw; i += nthreads) {
        dk[i] = sk[i];
        dv[i] = sv[i];
    }
}

// Pool summary row b with a 256-thread workgroup (thread t).  Every thread of
// a wave must call it (wave reduction); waves h >= H do nothing.  When
// lds_row is given, the stored row is also written there (same bits).
template <bool F16>
__device__ inline void pool_row(const UpdateArgs &a, int64_t b, int t, void *lds_row = nullptr)
{
    const int h = t >> 6;
    const int j = t & 63;
    const int half = a.D >> 1;
    if (h >= a.H)
        return;                       // whole waves only
    const bool act = j < half;
    const size_t row = (size_t)a.H * a.D;
    const size_t e_lo = (size_t)h * a.D + j;
    const size_t e_hi = e_lo + half;

    double lo = 0.0, hi = 0.0;
    if (act) {
        double s_lo = 0.0, s_hi = 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t tok = 4 * b + r;
            // Rows being appended by this same launch are read from their source.
            const bool fresh = a.new_idx_row && tok >= a.pos && tok < a.pos + a.n_new;
            const void *src = fresh ? a.new_idx_row : a.idx_k;
            const size_t base = (size_t)(fresh ? tok - a.pos : tok) * row;
            s_lo += load_idx<F16>(src, base + e_lo);
            s_hi += load_idx<F16>(src, base + e_hi);
        }
        lo = s_lo * 0.25;
        hi = s_hi * 0.25;
    }
    double sq = lo * lo + hi * hi;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        sq += __shfl_xor(sq, o);
    if (!act)
        return;
    const double inv_r = 1.0 / sqrt(sq / (double)a.D + a.eps);
    const double y_lo = lo * inv_r * (double)a.gamma[j];
    const double y_hi = hi * inv_r * (double)a.gamma[j + half];
    const double phi = (double)(4 * b) * pow(a.theta, -2.0 * (double)j / (double)a.D);
    double sn, cs;
    sincos(phi, &sn, &cs);
    const double o_lo = y_lo * cs - y_hi * sn;
    const double o_hi = y_lo * sn + y_hi * cs;
    const size_t dst = (size_t)b * row;
    if constexpr (F16) {
        uint16_t *sm = (uint16_t *)a.summary;
        const uint16_t v_lo = f64_to_f16_rne(o_lo), v_hi = f64_to_f16_rne(o_hi);
        sm[dst + e_lo] = v_lo;
        sm[dst + e_hi] = v_hi;
        if (lds_row) {
            ((uint16_t *)lds_row)[e_lo] = v_lo;
            ((uint16_t *)lds_row)[e_hi] = v_hi;
        }
    } else {
        float *sm = (float *)a.summary;
        sm[dst + e_lo] = (float)o_lo;
        sm[dst + e_hi] = (float)o_hi;
        if (lds_row) {
            ((float *)lds_row)[e_lo] = (float)o_lo;
            ((float *)lds_row)[e_hi] = (float)o_hi;
        }
    }
}

}  // namespace qsa
