"""CPU oracle of the QSA decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and it
never stands in for the GPU library.

Every function is a thin numpy/ctypes wrapper over ``qsa_oracle.c`` (plain C,
IEEE double throughout), plus the host-side watermark logic of the pooled-key
cache.  The method follows the public Qiita post no.10 by "ariera"
("第10回 EVO-X2（Ryzen AI Max+ 395 / 128GB）+ Qwen3.8-Flash-Next用のllama.cpp改造で
長コンテキストのTGを高速化した話"), sections "QSA indexer", "incremental
pooled-key cache（COMMON-004）", "selected QSA K/V gather（COMMON-005）" and
"block-domain top-k（COMMON-006）実装は見送り".  The readings taken where the
post is silent are listed at the top of ``qsa_oracle.c``.

Pins (checked by the CPU tests, none of them a re-typing of this code):
  pool / RMSNorm  -- closed-form worked example, scale invariance, the
                     mean-square identity, gamma acting per element;
  RoPE            -- p = 0 identity, complex-exponential special case,
                     pair-norm preservation, R(a)R(b) = R(a+b);
  scores          -- one-hot weights reduce to numpy.dot, linearity,
                     Cauchy-Schwarz bound;
  top-k           -- exhaustive subset search on tiny inputs, numpy.lexsort,
                     hand-checked tie example;
  cells           -- closed-form count, the 2048 + 4 - 1 ceiling;
  attention       -- torch scaled_dot_product_attention in float64 when every
                     block is kept, one-cell / equal-rows / zero-query cases;
  watermark       -- incremental == full rebuild after every append, and
                     after invalidate / truncate;
  q8_0 quantise   -- power-of-two scales (every step exact: codes are the
                     rounded quotients), a hand-checked tie block, a zero
                     block, the half-scale error bound and the 127 ceiling;
  q8_0 attention  -- equals attend() when every value is a binary16, and
                     torch attention in float64 over the decoded values.
No function here is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
F16 = 1

_lib = None


def lib():
    """Load liboracle, compiling it first only if it has never been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        d, l, i = ctypes.c_double, ctypes.c_long, ctypes.c_int
        L.qsa_oracle_half_to_double.restype = d
        L.qsa_oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.qsa_oracle_double_to_half.restype = ctypes.c_uint16
        L.qsa_oracle_double_to_half.argtypes = [d]
        L.qsa_oracle_summary_row.argtypes = [P, i, i, i, l, P, d, d, P]
        L.qsa_oracle_rope.argtypes = [P, i, d, d, P]
        L.qsa_oracle_cache_update.argtypes = [P, P, i, i, i, l, l, P, d, d]
        L.qsa_oracle_q8_0_quantize.argtypes = [P, l, P, P]
        L.qsa_oracle_attend_q8_0.argtypes = [P, P, P, P, P, P, l, i, i, i, d, P]
        L.qsa_oracle_scores.argtypes = [P, i, l, i, i, P, P, P, P]
        L.qsa_oracle_topk.restype = l
        L.qsa_oracle_topk.argtypes = [P, l, l, P]
        L.qsa_oracle_cells.restype = l
        L.qsa_oracle_cells.argtypes = [P, l, l, P]
        L.qsa_oracle_attend.argtypes = [P, P, P, P, l, i, i, i, d, P]
        L.qsa_oracle_union_blocks.restype = l
        L.qsa_oracle_union_blocks.argtypes = [P, P, i, i, P, l]
        L.qsa_oracle_union_attend.argtypes = [P, P, P, P, P, P, i, i, i, i, i, d, P]
        L.qsa_oracle_threads.restype = i
        L.qsa_oracle_threads.argtypes = []
        L.qsa_oracle_set_threads.argtypes = [i]
        _lib = L
    return _lib


def threads():
    """OpenMP threads of the oracle's parallel loops (blocks, heads)."""
    return int(lib().qsa_oracle_threads())


def set_threads(n):
    lib().qsa_oracle_set_threads(int(n))


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"raw keys / summaries must be float16 or float32, got {a.dtype}")


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def half_to_double(bits):
    return lib().qsa_oracle_half_to_double(int(bits))


def double_to_half(x):
    return lib().qsa_oracle_double_to_half(float(x))


def summary_row(raw, b, gamma, eps, theta):
    """Unrounded (float64) summary of block b.  raw: [tokens, H, D]."""
    raw = np.ascontiguousarray(raw)
    _, H, D = raw.shape
    g = _c(gamma, np.float32)
    out = np.empty((H, D), np.float64)
    lib().qsa_oracle_summary_row(_p(raw), _dtype_code(raw), H, D, int(b), _p(g),
                                 float(eps), float(theta), _p(out))
    return out


def rope(x, pos, theta):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().qsa_oracle_rope(_p(x), x.shape[-1], float(pos), float(theta), _p(out))
    return out


def cache_update(raw, summary, b0, b1, gamma, eps, theta):
    """Rebuild stored summary rows [b0, b1) in place (raw-key dtype)."""
    assert raw.dtype == summary.dtype and raw.flags.c_contiguous and summary.flags.c_contiguous
    _, H, D = raw.shape
    assert summary.shape[1:] == (H, D) and b1 <= summary.shape[0] and 4 * b1 <= raw.shape[0]
    g = _c(gamma, np.float32)
    lib().qsa_oracle_cache_update(_p(raw), _p(summary), _dtype_code(raw), H, D,
                                  int(b0), int(b1), _p(g), float(eps), float(theta))


def full_summaries(raw, nb, gamma, eps, theta):
    _, H, D = raw.shape
    s = np.zeros((max(nb, 1), H, D), raw.dtype)
    cache_update(np.ascontiguousarray(raw), s, 0, nb, gamma, eps, theta)
    return s[:nb]


def scores(summary, nb, q_idx, w, with_scale=False):
    summary = np.ascontiguousarray(summary)
    _, H, D = summary.shape
    q = _c(q_idx, np.float32)
    ww = _c(w, np.float32)
    assert q.size == H * D and ww.size == H
    s = np.empty(max(nb, 0), np.float64)
    a = np.empty(max(nb, 0), np.float64) if with_scale else None
    lib().qsa_oracle_scores(_p(summary), _dtype_code(summary), int(nb), H, D, _p(q), _p(ww),
                            _p(s), _p(a) if a is not None else None)
    return (s, a) if with_scale else s


def topk(s, k):
    s = _c(s, np.float64)
    nb = s.shape[0]
    sel = np.empty(max(min(k, nb), 1), np.int32)
    kb = lib().qsa_oracle_topk(_p(s), nb, int(k), _p(sel))
    return sel[:kb].copy()


def cells(sel, n):
    sel = _c(sel, np.int32)
    out = np.empty(4 * sel.shape[0] + 4, np.int32)
    nc = lib().qsa_oracle_cells(_p(sel), sel.shape[0], int(n), _p(out))
    return out[:nc].copy()


def attend(q, K, V, cell_ids, scale=None):
    """q: [Hq, Dh] fp32; K, V: [tokens, Hkv, Dh] float16; returns [Hq, Dh] float64."""
    q = _c(q, np.float32)
    Hq, Dh = q.shape
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    assert K.dtype == np.float16 and V.dtype == np.float16
    Hkv = K.shape[1]
    c = _c(cell_ids, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    out = np.empty((Hq, Dh), np.float64)
    lib().qsa_oracle_attend(_p(q), _p(K.view(np.uint16)), _p(V.view(np.uint16)), _p(c),
                            c.shape[0], Hq, Hkv, Dh, float(scale), _p(out))
    return out


def _sel_matrix(sels):
    nq = len(sels)
    kb = max(1, max(len(x) for x in sels))
    m = np.zeros((nq, kb), np.int32)
    k = np.zeros(nq, np.int32)
    for i, x in enumerate(sels):
        m[i, :len(x)] = x
        k[i] = len(x)
    return m, k, kb


def union_blocks(sels):
    """Ascending union of the queries' ascending block-id lists."""
    m, k, kb = _sel_matrix(sels)
    cap = int(k.sum()) + 1
    out = np.empty(cap, np.int32)
    nu = lib().qsa_oracle_union_blocks(_p(m), _p(k), len(sels), kb, _p(out), cap)
    assert nu >= 0
    return out[:nu].copy()


def union_attend(q, K, V, sels, n, scale=None):
    """Grouped-union attention of a group of queries (a reading: each query
    attends over the union of the group's cells with the others masked).
    q: [nq, Hq, Dh] fp32; sels: list of ascending id arrays; n: tokens seen
    per query.  Returns [nq, Hq, Dh] float64."""
    q = _c(q, np.float32)
    nq, Hq, Dh = q.shape
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    assert K.dtype == np.float16 and V.dtype == np.float16
    Hkv = K.shape[1]
    m, k, kb = _sel_matrix(sels)
    nn = _c(n, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    out = np.empty((nq, Hq, Dh), np.float64)
    lib().qsa_oracle_union_attend(_p(q), _p(K.view(np.uint16)), _p(V.view(np.uint16)), _p(m), _p(k), _p(nn),
                                  nq, kb, Hq, Hkv, Dh, float(scale), _p(out))
    return out


def q8_0_quantize(x):
    """q8_0 of a float16 array whose last axis is a multiple of 32: returns
    (codes int8, same shape; scales as binary16 bits, last axis / 32)."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    assert x.shape[-1] % 32 == 0
    nblk = x.size // 32
    codes = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), np.uint16)
    lib().qsa_oracle_q8_0_quantize(_p(x.view(np.uint16)), nblk, _p(codes), _p(d))
    return codes, d


def q8_0_values(codes, d):
    """code * scale in float64 (exact), same shape as codes."""
    c = np.asarray(codes, np.float64)
    s = np.asarray(d, np.uint16).view(np.float16).astype(np.float64)
    return c * np.repeat(s, 32, axis=-1)


def attend_q8_0(q, Kc, Kd, Vc, Vd, cell_ids, scale=None):
    """attend() over a q8_0 cache: Kc, Vc [tokens, Hkv, Dh] int8 codes;
    Kd, Vd [tokens, Hkv, Dh/32] binary16 scale bits.  Returns [Hq, Dh] float64."""
    q = _c(q, np.float32)
    Hq, Dh = q.shape
    Kc, Vc = _c(Kc, np.int8), _c(Vc, np.int8)
    Kd, Vd = _c(Kd, np.uint16), _c(Vd, np.uint16)
    Hkv = Kc.shape[1]
    assert Dh % 32 == 0 and Kd.shape[-1] == Dh // 32 and Vd.shape == Kd.shape
    c = _c(cell_ids, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    out = np.empty((Hq, Dh), np.float64)
    lib().qsa_oracle_attend_q8_0(_p(q), _p(Kc), _p(Kd), _p(Vc), _p(Vd), _p(c), c.shape[0],
                                 Hq, Hkv, Dh, float(scale), _p(out))
    return out


def n_cells(n, k_blocks):
    """|C| = 4 * min(K, floor(n/4)) + n mod 4."""
    return 4 * min(k_blocks, n // 4) + n % 4


class OracleLayer:
    """One sequence x one QSA layer, held in host memory.

    Holds the raw indexer keys, the pooled summary cache and its watermark
    ``valid`` (rows [0, valid) are trusted), the K/V cache and the token
    count.  ``step`` follows the incremental pooled-key cache: only rows
    [valid, n/4) are rebuilt before scoring [post 10, "incremental pooled-key
    cache（COMMON-004）"].  ``invalidate`` (state load / distrust) and
    ``truncate`` (sequence edit) lower the watermark so that the next step
    rebuilds what is no longer trusted.
    """

    def __init__(self, raw, K, V, gamma, eps, theta, n_tokens, k_blocks, valid=0):
        self.raw = np.ascontiguousarray(raw)
        self.K = np.ascontiguousarray(K)
        self.V = np.ascontiguousarray(V)
        cap, H, D = self.raw.shape
        self.summary = np.zeros((cap // 4, H, D), self.raw.dtype)
        self.gamma = _c(gamma, np.float32)
        self.eps, self.theta = float(eps), float(theta)
        self.n = int(n_tokens)
        self.valid = int(valid)
        self.k_blocks = int(k_blocks)

    def rebuild(self):
        nb = self.n // 4
        if self.valid < nb:
            cache_update(self.raw, self.summary, self.valid, nb, self.gamma, self.eps, self.theta)
        self.valid = nb

    def invalidate(self, pos):
        self.valid = min(self.valid, int(pos) // 4)

    def truncate(self, pos):
        self.n = min(self.n, int(pos))
        self.invalidate(pos)

    def append(self, raw_row, k_row, v_row):
        t = self.n
        self.raw[t] = raw_row
        self.K[t] = k_row
        self.V[t] = v_row
        self.n = t + 1

    def step(self, raw_row, k_row, v_row, q_idx, w, q, scale=None):
        """Append one token, refresh the cache, score, select and attend."""
        self.append(raw_row, k_row, v_row)
        self.rebuild()
        nb = self.n // 4
        s = scores(self.summary, nb, q_idx, w)
        sel = topk(s, self.k_blocks)
        c = cells(sel, self.n)
        out = attend(q, self.K, self.V, c, scale)
        return {"scores": s, "sel": sel, "cells": c, "out": out}
