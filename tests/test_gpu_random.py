"""Seeded random configurations through the multi-query and decode paths,
each against the CPU oracle: contexts from a few tokens to 70k (every tile
list length the top-k picks, tail-only and keep-every-block steps), 1-4
tokens per call, every alignment to the 4-token block, indexer and GQA
shapes.  The configuration list is fixed by the seed, so a failure names
its case and reruns the same way."""
import numpy as np
import pytest

from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W
from test_gpu_multi import _check, _host_tokens, _multi, _oracle_take
from parity import check_summaries

pytestmark = pytest.mark.gpu

_SHAPES = [  # idx_heads, idx_dim, idx_f16, q_heads, kv_heads, head_dim, top_k_tokens
    (4, 128, True, 16, 2, 256, 2048),
    (1, 64, False, 4, 1, 64, 256),
    (1, 128, True, 8, 2, 128, 512),
    (4, 64, False, 2, 2, 64, 1024),
]


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    for i in range(n):
        shape = _SHAPES[int(rng.integers(len(_SHAPES)))]
        n0 = int(rng.choice([int(rng.integers(0, 64)), int(rng.integers(64, 4096)),
                             int(rng.integers(4096, 70000))]))
        yield i, shape, n0, int(rng.integers(1, 5)), int(rng.integers(1, 3))


@pytest.mark.parametrize("i,shape,n0,n_q,calls", list(_cases()), ids=[f"case{c[0]}" for c in _cases()])
def test_random_multi_then_decode(i, shape, n0, n_q, calls):
    import torch
    Hi, Di, f16, Hq, Hkv, Dh, topk = shape
    w = with_size(W.CTX64K, n0=n0, steps=n_q * calls + 1, idx_heads=Hi, idx_dim=Di, idx_f16=f16,
                  q_heads=Hq, kv_heads=Hkv, head_dim=Dh, top_k_tokens=topk)
    print(f"case {i}: shape {shape} n0={n0} n_q={n_q} calls={calls}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    step = 0
    for _ in range(calls):
        p = g.state.n_tokens
        toks = _host_tokens(w, range(p, p + n_q), [0] * n_q, range(step, step + n_q))
        res = _multi(g, toks)
        for j in range(n_q):
            _oracle_take(o.L, toks, j)
            _check(j, o.L, toks, res, w.k_blocks, stats)
        step += n_q
    # then one plain decode step
    p = g.state.n_tokens
    toks = _host_tokens(w, [p], [0], [step])
    raw, kr, vr, qi, wt, q = (torch.from_numpy(x).cuda() for x in toks)
    g.qsa.qsa_decode_step(g.desc, g.buf.cache, g.state, raw[0], kr[0], vr[0], g.gamma, qi[0], wt[0],
                          q[0], g.out, g.sel, g.scores, g.ws)
    torch.cuda.synchronize()
    _oracle_take(o.L, toks, 0)
    nb = g.state.n_tokens // 4
    kb = min(w.k_blocks, nb)
    sel = np.full((1, w.k_blocks), -1, np.int32)
    sel[0, :kb] = g.sel[:kb].cpu().numpy()
    sc = g.scores[:nb].cpu().numpy()[None] if nb > 0 else np.zeros((1, 1), np.float32)
    _check(0, o.L, toks, (g.out.cpu().numpy().astype(np.float64)[None], sel, sc, nb), w.k_blocks, stats)
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])
    print(f"  {stats}")
