"""Synthetic QSA decode workloads: shapes, seeds and seeded cache fills.

Shapes follow the decode configurations measured on post 10 (ariera,
qiita.com): inputs of 61,789 / 126,253 / 255,181 tokens for the 64k / 128k /
256k contexts (section "検証環境" and the appendix table of input sizes), f16
K/V, indexer top-k 2048 tokens with compression 4 (section "QSA indexer"), and
12 QSA layers per token (section "128kと256kを比較してみる").  The
post's long Japanese documents are not available; seeded synthetic data of
the same shapes stands in for them.  Distributions: raw indexer keys, K, V,
q_idx and q ~ N(0,1) (Irwin-Hall approximation, see csrc/qsagen_core.h),
w ~ U(0,1), gamma ~ U(0.5,1.5).

Nothing here computes any part of the attention method.
"""
from dataclasses import dataclass, field

import numpy as np

from . import (BASE_SEED, KIND_GAMMA, KIND_K, KIND_Q, KIND_QIDX, KIND_RAW, KIND_V, KIND_W,
               dev_normal_, dev_unit_, host_normal, host_rows, host_unit, tensor_id)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    layers: int
    n0: int                 # tokens already in the cache before the first decode step
    steps: int              # decode steps per layer
    idx_heads: int
    idx_dim: int
    idx_f16: bool
    q_heads: int
    kv_heads: int
    head_dim: int
    top_k_tokens: int
    rms_eps: float = float(np.float32(1e-6))   # the value the library receives (fp32)
    rope_theta: float = 1e4

    @property
    def seed(self):
        return BASE_SEED + self.cfg_id

    @property
    def k_blocks(self):
        return self.top_k_tokens // 4

    def capacity(self, extra_steps=0):
        n = self.n0 + self.steps + extra_steps
        return (n + 3) // 4 * 4

    @property
    def idx_row(self):
        return (self.idx_heads, self.idx_dim)

    @property
    def kv_row(self):
        return (self.kv_heads, self.head_dim)


TINY = Workload("tiny-4k", 0, 1, 4096, 32, 1, 64, False, 4, 1, 64, 256)
CTX64K = Workload("qsa-64k", 1, 1, 61789, 128, 4, 128, True, 16, 2, 256, 2048)
CTX128K = Workload("qsa-128k", 2, 1, 126253, 128, 4, 128, True, 16, 2, 256, 2048)
CTX256K = Workload("qsa-256k-12layers", 3, 12, 255181, 64, 4, 128, True, 16, 2, 256, 2048)
WORKLOADS = {w.name: w for w in (TINY, CTX64K, CTX128K, CTX256K)}

# Batched decode + prefill chunk, same layer shapes: eight sequences of mixed
# context (16k / 32k / 64k / 128k / 256k inputs, the last three repeated), and
# one 1024-token chunk (the post's ubatch size) at the 128k input size.
BATCH_CONTEXTS = (16381, 29453, 61789, 126253, 255181, 16381, 29453, 61789)
BATCH = Workload("qsa-batch8-mixed", 4, 1, 16381, 64, 4, 128, True, 16, 2, 256, 2048)
CHUNK128K = Workload("qsa-chunk1024-128k", 5, 1, 126253, 1024, 4, 128, True, 16, 2, 256, 2048)


def ids(layer, seq=0):
    return {k: tensor_id(k, layer=layer, seq=seq) for k in (KIND_RAW, KIND_K, KIND_V, KIND_GAMMA)}


# ------------------------------------------------------------------ host side
def host_gamma(w: Workload, layer, seq=0):
    return host_unit((w.idx_dim,), w.seed, tensor_id(KIND_GAMMA, layer=layer, seq=seq), offset=0.5)


def host_raw_rows(w: Workload, rows, layer, seq=0):
    dt = np.float16 if w.idx_f16 else np.float32
    return host_rows(rows, w.idx_row, w.seed, tensor_id(KIND_RAW, layer=layer, seq=seq), dtype=dt)


def host_kv_rows(w: Workload, rows, layer, seq=0):
    k = host_rows(rows, w.kv_row, w.seed, tensor_id(KIND_K, layer=layer, seq=seq), dtype=np.float16)
    v = host_rows(rows, w.kv_row, w.seed, tensor_id(KIND_V, layer=layer, seq=seq), dtype=np.float16)
    return k, v


def host_step_inputs(w: Workload, layer, step, seq=0):
    """Per-step query inputs: q_idx [H_i, D_i], w [H_i], q [Hq, Dh] (fp32)."""
    q_idx = host_normal(w.idx_row, w.seed, tensor_id(KIND_QIDX, layer=layer, step=step, seq=seq))
    wt = host_unit((w.idx_heads,), w.seed, tensor_id(KIND_W, layer=layer, step=step, seq=seq))
    q = host_normal((w.q_heads, w.head_dim), w.seed, tensor_id(KIND_Q, layer=layer, step=step, seq=seq))
    return q_idx, wt, q


# Correlated queries: consecutive tokens of one passage tend to choose
# overlapping blocks (the case a grouped-union prefill serves); here the
# indexer query of step s is sqrt(rho) B + sqrt(1 - rho) N_s, B one seeded
# N(0,1) tensor per layer and N_s step s's own q_idx (computed in double,
# rounded once to fp32).
CORR_BASE_STEP = (1 << 24) - 1          # step slot of the shared tensor B


def host_correlated_q_idx(w: Workload, layer, first_step, steps, rho, seq=0):
    """[steps, H_i, D_i] fp32 correlated indexer queries (see above)."""
    base = host_normal(w.idx_row, w.seed, tensor_id(KIND_QIDX, layer=layer, step=CORR_BASE_STEP, seq=seq))
    out = np.empty((steps,) + w.idx_row, np.float32)
    for s in range(steps):
        noise = host_step_inputs(w, layer, first_step + s, seq)[0]
        out[s] = (np.sqrt(rho) * base.astype(np.float64) +
                  np.sqrt(1.0 - rho) * noise.astype(np.float64)).astype(np.float32)
    return out


# ---------------------------------------------------------------- device side
def poison_(t):
    """Fill with NaN so that a row read before it is written shows up."""
    t.fill_(float("nan"))
    return t


def dev_fill_layer_(w: Workload, buf, layer, n_filled, seq=0, stream=None):
    """Seeded rows [0, n_filled) of raw keys, K and V; NaN beyond."""
    import torch  # noqa: F401
    rl_i = w.idx_heads * w.idx_dim
    rl_kv = w.kv_heads * w.head_dim
    for t, kind, rl in ((buf.idx_k, KIND_RAW, rl_i), (buf.k, KIND_K, rl_kv), (buf.v, KIND_V, rl_kv)):
        head = t[:n_filled]
        if n_filled:
            dev_normal_(head.view(-1), w.seed, tensor_id(kind, layer=layer, seq=seq), 0, stream)
        if n_filled < t.shape[0]:
            poison_(t[n_filled:])
    poison_(buf.summary)


def dev_gamma(w: Workload, layer, seq=0, device="cuda", stream=None):
    import torch
    g = torch.empty(w.idx_dim, dtype=torch.float32, device=device)
    return dev_unit_(g, w.seed, tensor_id(KIND_GAMMA, layer=layer, seq=seq), 0, 0.5, stream)


@dataclass
class StepInputs:
    """Per-step device inputs for `steps` consecutive steps of one layer."""
    raw: object = None      # [steps, H_i, D_i]
    k: object = None        # [steps, Hkv, Dh] f16
    v: object = None
    q_idx: object = None    # [steps, H_i, D_i] fp32
    w: object = None        # [steps, H_i] fp32
    q: object = None        # [steps, Hq, Dh] fp32
    extra: dict = field(default_factory=dict)


def dev_step_inputs(w: Workload, layer, first_step, steps, seq=0, device="cuda", stream=None):
    """Rows n0 + first_step ... of the cache streams, and the per-step queries."""
    import torch
    dt = torch.float16 if w.idx_f16 else torch.float32
    rl_i = w.idx_heads * w.idx_dim
    rl_kv = w.kv_heads * w.head_dim
    pos0 = w.n0 + first_step
    si = StepInputs()
    si.raw = torch.empty((steps,) + w.idx_row, dtype=dt, device=device)
    si.k = torch.empty((steps,) + w.kv_row, dtype=torch.float16, device=device)
    si.v = torch.empty_like(si.k)
    dev_normal_(si.raw.view(-1), w.seed, tensor_id(KIND_RAW, layer=layer, seq=seq), pos0 * rl_i, stream)
    dev_normal_(si.k.view(-1), w.seed, tensor_id(KIND_K, layer=layer, seq=seq), pos0 * rl_kv, stream)
    dev_normal_(si.v.view(-1), w.seed, tensor_id(KIND_V, layer=layer, seq=seq), pos0 * rl_kv, stream)
    si.q_idx = torch.empty((steps,) + w.idx_row, dtype=torch.float32, device=device)
    si.w = torch.empty((steps, w.idx_heads), dtype=torch.float32, device=device)
    si.q = torch.empty((steps, w.q_heads, w.head_dim), dtype=torch.float32, device=device)
    for s in range(steps):
        st = first_step + s
        dev_normal_(si.q_idx[s].view(-1), w.seed, tensor_id(KIND_QIDX, layer=layer, step=st, seq=seq), 0, stream)
        dev_unit_(si.w[s], w.seed, tensor_id(KIND_W, layer=layer, step=st, seq=seq), 0, 0.0, stream)
        dev_normal_(si.q[s].view(-1), w.seed, tensor_id(KIND_Q, layer=layer, step=st, seq=seq), 0, stream)
    return si
