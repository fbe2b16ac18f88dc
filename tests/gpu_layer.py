"""Test-side set-up of one GPU layer and its CPU-oracle mirror.

GpuLayer drives the HIP library through its binding; OracleMirror holds the
same seeded inputs on the host (regenerated with the host generator, never
copied back from the GPU) and steps the CPU oracle.
"""
import dataclasses

import numpy as np

import oracle
from qsagen import workloads as W


def with_size(w, n0=None, steps=None, **kw):
    kw = dict(kw)
    if n0 is not None:
        kw["n0"] = n0
    if steps is not None:
        kw["steps"] = steps
    return dataclasses.replace(w, **kw)


class GpuLayer:
    def __init__(self, w, layer=0, seq=0, prefill=True, gamma_seq=None, planted=None):
        import torch
        import sparse_attention_decode_cache_amd as qsa
        self.qsa = qsa
        self.w = w
        self.layer = layer
        self.cap = w.capacity()
        self.desc = qsa.make_desc(w.idx_heads, w.idx_dim, qsa.QSA_F16 if w.idx_f16 else qsa.QSA_F32,
                                  w.q_heads, w.kv_heads, w.head_dim, w.top_k_tokens,
                                  w.rms_eps, w.rope_theta)
        self.buf = qsa.LayerBuffers(self.desc, self.cap)
        W.dev_fill_layer_(w, self.buf, layer, w.n0, seq)
        if planted is not None:
            import planted as PL
            PL.apply_device(planted, self.buf.idx_k)
        self.gamma = W.dev_gamma(w, layer, seq if gamma_seq is None else gamma_seq)
        self.ws = qsa.workspace(self.desc, self.cap)
        self.state = qsa.qsa_seq_state(w.n0, 0)
        if prefill:
            qsa.qsa_cache_update(self.desc, self.buf.cache, self.gamma, 0, w.n0 // 4)
            self.state.n_valid_blocks = w.n0 // 4
        self.inp = W.dev_step_inputs(w, layer, 0, max(w.steps, 1), seq)
        if planted is not None:
            self.inp.q_idx[:] = torch.from_numpy(planted.q_idx).cuda()
            self.inp.w[:] = torch.from_numpy(planted.w).cuda()
        self.out = torch.empty((w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        self.sel = torch.empty(w.k_blocks, dtype=torch.int32, device="cuda")
        self.scores = torch.empty(self.cap // 4, dtype=torch.float32, device="cuda")

    def path(self):
        """How the last selecting decode step chose its blocks (the low byte of
        the workspace's status word): QSA_PATH_HIST or QSA_PATH_FULL."""
        o = self.qsa.QSA_DECODE_STATUS_OFFSET
        return int(self.ws[o:o + 8].cpu().numpy().view("<u8")[0] & 0xFF)

    def step(self, s):
        q = self.qsa
        q.qsa_decode_step(self.desc, self.buf.cache, self.state, self.inp.raw[s], self.inp.k[s],
                          self.inp.v[s], self.gamma, self.inp.q_idx[s], self.inp.w[s], self.inp.q[s],
                          self.out, self.sel, self.scores, self.ws)
        n = self.state.n_tokens
        nb = n // 4
        return {"n": n, "nb": nb, "out": self.out.cpu().numpy().astype(np.float64),
                "sel": self.sel[:min(self.w.k_blocks, nb)].cpu().numpy(),
                "scores": self.scores[:nb].cpu().numpy()}


class OracleMirror:
    def __init__(self, w, layer=0, seq=0, gamma_seq=None, planted=None):
        self.w = w
        self.layer = layer
        cap = w.capacity()
        dt = np.float16 if w.idx_f16 else np.float32
        raw = np.zeros((cap,) + w.idx_row, dt)
        K = np.zeros((cap,) + w.kv_row, np.float16)
        V = np.zeros_like(K)
        rows = np.arange(w.n0)
        raw[:w.n0] = W.host_raw_rows(w, rows, layer, seq)
        self.planted = planted
        if planted is not None:
            import planted as PL
            PL.apply_host(planted, raw)
        K[:w.n0], V[:w.n0] = W.host_kv_rows(w, rows, layer, seq)
        self.gamma = W.host_gamma(w, layer, seq if gamma_seq is None else gamma_seq)
        self.L = oracle.OracleLayer(raw, K, V, self.gamma, w.rms_eps, w.rope_theta, w.n0, w.k_blocks)
        self.L.rebuild()
        self.seq = seq

    def step(self, s):
        w = self.w
        pos = w.n0 + s
        assert self.L.n == pos
        raw_row = W.host_raw_rows(w, [pos], self.layer, self.seq)[0]
        k_row, v_row = (x[0] for x in W.host_kv_rows(w, [pos], self.layer, self.seq))
        q_idx, wt, q = W.host_step_inputs(w, self.layer, s, self.seq)
        if self.planted is not None:
            q_idx, wt = self.planted.q_idx, self.planted.w
        r = self.L.step(raw_row, k_row, v_row, q_idx, wt, q)
        nb = self.L.n // 4
        r["scale"] = oracle.scores(self.L.summary, nb, q_idx, wt, with_scale=True)[1]
        r["q"] = q
        return r
