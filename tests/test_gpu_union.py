"""Grouped-union prefill attention (qsa_chunk_step_grouped, a reading of
post 10's "QSA grouped-union") on the GPU: the same chunk through
qsa_chunk_step and through the grouped path must choose the same blocks
(bit for bit) and give the same outputs to the attention tolerance, and the
grouped outputs must match the oracle's grouped-union attention of each
group (its queries' own cells, the others masked) on the chosen blocks.
Queries are correlated (consecutive tokens choose overlapping blocks) or
independent; groups are min(64 / G, 32) queries, the last one partial."""
import numpy as np
import pytest

import oracle
from gpu_layer import GpuLayer, OracleMirror, with_size
from parity import ATTN_ATOL
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def union_group(G, nb_last):
    """Queries per group, the rule qsa_chunk_step_grouped documents: min(64 /
    G, 32), fewer while their bitmaps (ceil(nb_last / 32) words per query,
    plus 8 words) exceed 128 KB."""
    qg = min(64 // G, 32)
    while qg > 1 and 4 * (qg * ((nb_last + 31) // 32) + 8) > 128 * 1024:
        qg -= 1
    return qg


def _run(g, n_q, grouped, q_idx=None):
    import torch
    qsa = g.qsa
    w = g.w
    if q_idx is not None:
        g.inp.q_idx[:n_q] = torch.from_numpy(q_idx).cuda()
    nb_last = (g.state.n_tokens + n_q) // 4
    ws = qsa.chunk_workspace(g.desc, g.cap, n_q)
    out = torch.full((n_q, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((n_q, w.k_blocks), -7, dtype=torch.int32, device="cuda")
    scores = torch.full((n_q, max(nb_last, 1)), float("nan"), dtype=torch.float32, device="cuda")
    inp = g.inp
    f = qsa.qsa_chunk_step_grouped if grouped else qsa.qsa_chunk_step
    f(g.desc, g.buf.cache, g.state, n_q, inp.raw[:n_q], inp.k[:n_q], inp.v[:n_q], g.gamma, inp.q_idx[:n_q],
      inp.w[:n_q], inp.q[:n_q], out, sel, scores, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), sel.cpu().numpy(), scores.cpu().numpy()


@pytest.mark.parametrize("base,n0,n_q,rho", [
    (W.CTX64K, 61789, 64, 0.95),      # G = 8: groups of 8 (four row tiles), correlated
    (W.CTX64K, 61789, 37, None),      # independent queries, a partial last group
    (W.TINY, 4096, 40, 0.9),          # G = 4: groups of 16, K = 64
    (W.TINY, 150, 23, None),          # every block kept (no selection), partial group
], ids=["64k-corr", "64k-iid", "tiny-corr", "tiny-keepall"])
def test_grouped_union_matches_per_query_and_oracle(base, n0, n_q, rho):
    w = with_size(base, n0=n0, steps=n_q)
    print(f"union chunk {w.name}: n0={n0} n_q={n_q} rho={rho}", flush=True)
    q_idx = None if rho is None else W.host_correlated_q_idx(w, 0, 0, n_q, rho)
    a = GpuLayer(w)
    b = GpuLayer(w)
    out_a, sel_a, sc_a = _run(a, n_q, False, q_idx)
    out_b, sel_b, sc_b = _run(b, n_q, True, q_idx)
    assert np.array_equal(sel_a, sel_b)
    assert np.array_equal(sc_a.view(np.uint32), sc_b.view(np.uint32)) or np.isnan(sc_a).all()
    err = float(np.max(np.abs(out_a - out_b)))
    assert err <= 1e-4, err
    # the oracle: K / V rows after the chunk, grouped-union attention per group
    o = OracleMirror(w)
    for s in range(n_q):
        o.L.append(*(lambda r, kv: (r, kv[0][0], kv[1][0]))(
            W.host_raw_rows(w, [n0 + s], 0)[0], W.host_kv_rows(w, [n0 + s], 0)))
    G = w.q_heads // w.kv_heads
    qg = union_group(G, (n0 + n_q) // 4)
    q_all = np.stack([W.host_step_inputs(w, 0, s)[2] for s in range(n_q)])
    worst = 0.0
    sizes = []
    for j in range(0, n_q, qg):
        idx = list(range(j, min(n_q, j + qg)))
        n = [n0 + i + 1 for i in idx]
        sels = [sel_b[i, :min(w.k_blocks, n[k] // 4)] for k, i in enumerate(idx)]
        ref = oracle.union_attend(q_all[idx], o.L.K, o.L.V, sels, n)
        worst = max(worst, float(np.max(np.abs(out_b[idx] - ref))))
        sizes.append(len(oracle.union_blocks(sels)))
    print(f"  max |grouped - oracle| {worst:.2e}; union blocks per group: mean {np.mean(sizes):.0f} "
          f"(K = {w.k_blocks}, {qg} queries per group)")
    assert worst <= ATTN_ATOL, worst
    if rho is not None and w.k_blocks < n0 // 4:
        # correlated: the group's choices overlap (the union is well below qg K)
        assert np.mean(sizes) < 0.9 * qg * w.k_blocks, sizes


@pytest.mark.parametrize("q_heads,kv_heads,head_dim,n_q", [
    (2, 2, 128, 45),        # G = 1: groups of 32 queries, two row tiles
    (4, 4, 256, 33),        # G = 1 at 256 dims
    (4, 2, 64, 70),         # G = 2: groups of 32, four row tiles
    (8, 2, 128, 19),        # G = 4: groups of 16, a partial group
    (16, 2, 64, 23)])       # G = 8 at 64 dims
def test_grouped_union_shapes(q_heads, kv_heads, head_dim, n_q):
    """GQA groups of 1 .. 8 heads and head dims 64 / 128 / 256 through the
    grouped path (groups of one, two and four matrix-core row tiles), on
    correlated queries: outputs against the per-query path, selections bit
    for bit."""
    w = with_size(W.CTX64K, n0=3001, steps=n_q, q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim)
    print(f"union shapes {q_heads}/{kv_heads}x{head_dim}: n_q={n_q} "
          f"({union_group(q_heads // kv_heads, (3001 + n_q) // 4)} queries per group)", flush=True)
    q_idx = W.host_correlated_q_idx(w, 0, 0, n_q, 0.95)
    out_a, sel_a, _ = _run(GpuLayer(w), n_q, False, q_idx)
    out_b, sel_b, _ = _run(GpuLayer(w), n_q, True, q_idx)
    assert np.array_equal(sel_a, sel_b)
    assert np.isfinite(out_b).all()
    err = float(np.max(np.abs(out_a - out_b)))
    assert err <= 1e-4, err
