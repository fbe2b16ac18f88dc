"""Prefill chunk (qsa_chunk_step) against the CPU oracle: token i of a chunk
must give what the i-th of as many decode steps in a row gives -- its scores
over the blocks completed by then (a causal block mask), its top-k, and its
attention -- and the pooled cache after the chunk must equal the oracle's.

The oracle runs the plain per-step definition; the GPU scores all queries of
the chunk in one matrix-core GEMM, selects per query and attends per query."""
import numpy as np
import pytest

import oracle
from parity import check_attention, check_scores, check_summaries, check_topk
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _chunk(g, n_q, with_scores=True):
    """Run tokens 0 .. n_q-1 of g's step inputs as one chunk."""
    import torch
    qsa = g.qsa
    w = g.w
    n0 = g.state.n_tokens
    nb_last = (n0 + n_q) // 4
    ws = qsa.chunk_workspace(g.desc, g.cap, n_q)
    out = torch.full((n_q, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((n_q, w.k_blocks), -7, dtype=torch.int32, device="cuda")
    scores = (torch.full((n_q, max(nb_last, 1)), float("nan"), dtype=torch.float32, device="cuda")
              if with_scores else None)
    inp = g.inp
    qsa.qsa_chunk_step(g.desc, g.buf.cache, g.state, n_q, inp.raw[:n_q], inp.k[:n_q], inp.v[:n_q],
                       g.gamma, inp.q_idx[:n_q], inp.w[:n_q], inp.q[:n_q], out, sel, scores, ws)
    torch.cuda.synchronize()
    assert (g.state.n_tokens, g.state.n_valid_blocks) == (n0 + n_q, nb_last)
    return (out.cpu().numpy().astype(np.float64), sel.cpu().numpy(),
            scores.cpu().numpy() if with_scores else None)


def _check_query(i, o, out, sel, scores, k_blocks, scored, stats):
    """Query i of the chunk against oracle step i (o has just taken it)."""
    ro = o.last
    n = o.L.n
    nb = n // 4
    kb = min(k_blocks, nb)
    assert np.all(sel[i, kb:] == -1), f"query {i}: slots past {kb} not -1"
    if scored:
        check_scores(scores[i, :nb], ro["scores"], ro["scale"])
        assert np.all(scores[i, nb:] == -np.inf), f"query {i}: masked scores not -inf"
    branch = check_topk(sel[i, :kb], ro["scores"], ro["scale"], k_blocks)
    stats[branch] += 1
    cells = oracle.cells(sel[i, :kb], n)
    assert len(cells) == oracle.n_cells(n, k_blocks)
    ref = oracle.attend(ro["q"], o.L.K, o.L.V, cells)
    stats["attn_err"] = max(stats["attn_err"], check_attention(out[i], ref))
    if branch == "exact":
        check_attention(out[i], ro["out"])


class _Mirror(OracleMirror):
    def step(self, s):
        self.last = super().step(s)
        return self.last


def _run_full(base, n0, n_q):
    """Every query of the chunk checked."""
    w = with_size(base, n0=n0, steps=n_q)
    print(f"chunk {w.name}: n0={n0} n_q={n_q} K={w.k_blocks}", flush=True)
    g = GpuLayer(w)
    o = _Mirror(w)
    nb_last = (n0 + n_q) // 4
    out, sel, scores = _chunk(g, n_q)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in range(n_q):
        o.step(i)
        _check_query(i, o, out, sel, scores, w.k_blocks, nb_last > w.k_blocks, stats)
    summ = g.buf.summary[:nb_last].cpu().numpy()
    ulp = check_summaries(summ, o.L.summary[:nb_last])
    print(f"  {stats} summary ulp diffs {ulp}")
    return stats


def test_chunk_crosses_top_k():
    """4 x 128 f16 indexer, 16/2 x 256 attention, K = 512 blocks: the first
    queries keep every block, the later ones select; 77 queries (a ragged
    query tile)."""
    st = _run_full(W.CTX64K, 2013, 77)
    assert st["exact"] + st["threshold"] == 77


def test_chunk_selects_every_query():
    st = _run_full(W.CTX64K, 9001, 130)
    assert st["exact"] + st["threshold"] == 130


def test_chunk_fp32_indexer():
    """1 x 64 fp32 indexer (summaries split into two f16 halves too), 4/1 x 64
    attention, K = 64 blocks."""
    st = _run_full(W.TINY, 4096, 48)
    assert st["exact"] + st["threshold"] == 48


def test_chunk_few_queries_split_and_merge():
    """6 queries: each query's tiles are split over many workgroups and merged."""
    st = _run_full(W.CTX64K, 20003, 6)
    assert st["exact"] + st["threshold"] == 6


def test_chunk_of_three_runs_the_multi_query_path():
    """3 queries (at most QSA_MAX_MULTI): the multi-query path, same results."""
    st = _run_full(W.CTX64K, 20003, 3)
    assert st["exact"] + st["threshold"] == 3


def test_chunk_single_query_matches_decode_step():
    """A chunk of one token is a decode step."""
    st = _run_full(W.CTX64K, 5001, 1)
    assert st["exact"] + st["threshold"] == 1


def test_chunk_from_empty_cache():
    """From position 0: the first queries see no block at all (tail only);
    nothing is scored while every query keeps all its blocks."""
    st = _run_full(W.TINY, 0, 45)
    assert st["exact"] == 45


def test_chunk_after_invalidation_rebuilds():
    """The watermark below the chunk start: the chunk pools the rows it
    distrusts again, with its own blocks."""
    w = with_size(W.CTX64K, n0=3001, steps=40)
    g = GpuLayer(w)
    g.qsa.qsa_state_invalidate(g.state, 1000)
    o = _Mirror(w)
    o.L.invalidate(1000)
    out, sel, scores = _chunk(g, 40)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in range(40):
        o.step(i)
        _check_query(i, o, out, sel, scores, w.k_blocks, True, stats)
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])


def test_chunk_128k_1024_queries_sampled():
    """The 1024-query chunk at 128k context (126,253 tokens, positions
    126,253 .. 127,276, 256 new blocks): sampled queries against the oracle
    at their own position, and every query's ids checked for validity."""
    w = with_size(W.CTX128K, n0=126253, steps=1024)
    n_q = 1024
    print(f"chunk {w.name}: n0={w.n0} n_q={n_q}", flush=True)
    g = GpuLayer(w)
    out, sel, scores = _chunk(g, n_q)
    assert np.isfinite(out).all()
    for i in range(n_q):
        nb = (w.n0 + i + 1) // 4
        row = sel[i]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < nb, f"query {i} ids"
    o = _Mirror(w)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    sample = [0, 1, 2, 3, 4, 255, 509, 510, 511, 777, 1020, 1021, 1022, 1023]
    for i in sample:
        # rows of the tokens before i, then token i as a decode step
        pos = w.n0 + i
        if o.L.n < pos:
            rows = np.arange(o.L.n, pos)
            o.L.raw[rows] = W.host_raw_rows(w, rows, 0)
            o.L.K[rows], o.L.V[rows] = W.host_kv_rows(w, rows, 0)
            o.L.n = pos
        o.step(i)
        _check_query(i, o, out, sel, scores, w.k_blocks, True, stats)
    print(f"  {stats}")
    # the oracle has now taken token 1023: its cache holds every block of the chunk
    nb_last = g.state.n_valid_blocks
    assert o.L.n // 4 == nb_last
    check_summaries(g.buf.summary[nb_last - 300:nb_last].cpu().numpy(), o.L.summary[nb_last - 300:nb_last])


@pytest.mark.parametrize("q_heads,kv_heads,head_dim,n_q", [
    (2, 2, 128, 21), (4, 2, 64, 37), (8, 2, 128, 19), (16, 2, 64, 23), (4, 4, 256, 17),
    (2, 2, 64, 5), (16, 2, 128, 7)])
def test_chunk_attention_shapes(q_heads, kv_heads, head_dim, n_q):
    """GQA groups of 1, 2, 4 and 8 heads, head dims 64 / 128 / 256; the last two
    cases have so few queries that each query is split and merged."""
    base = with_size(W.CTX64K, q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim)
    st = _run_full(base, 3001, n_q)
    assert st["exact"] + st["threshold"] == n_q


@pytest.mark.parametrize("idx_heads,idx_dim,idx_f16", [
    (1, 128, True), (4, 64, False), (1, 64, True), (1, 128, False), (4, 64, True)])
def test_chunk_indexer_shapes(idx_heads, idx_dim, idx_f16):
    """Indexer contractions of 64 .. 512 elements, f16 and fp32 summaries."""
    base = with_size(W.CTX64K, idx_heads=idx_heads, idx_dim=idx_dim, idx_f16=idx_f16)
    st = _run_full(base, 4001, 33)
    assert st["exact"] + st["threshold"] == 33


@pytest.mark.parametrize("idx_heads,idx_dim,n0,n_q", [
    (4, 128, 9001, 130), (1, 64, 4001, 33), (4, 64, 20003, 200)])
def test_chunk_without_scores_output_is_identical(idx_heads, idx_dim, n0, n_q):
    """Without the optional fp32 scores the score GEMM runs its keys-only
    instance (the one a caller that wants only the attention gets): the ids
    and outputs must be bit-identical to those of the run that writes scores
    (the keys are formed the same way in both), and that run is checked
    against the oracle."""
    base = with_size(W.CTX64K, idx_heads=idx_heads, idx_dim=idx_dim, idx_f16=True)
    w = with_size(base, n0=n0, steps=n_q)
    print(f"chunk {w.name}: n0={n0} n_q={n_q} with and without scores", flush=True)
    a = GpuLayer(w)
    out_a, sel_a, scores = _chunk(a, n_q, with_scores=True)
    b = GpuLayer(w)
    out_b, sel_b, _ = _chunk(b, n_q, with_scores=False)
    assert np.array_equal(sel_a, sel_b)
    assert np.array_equal(out_a, out_b)
    o = _Mirror(w)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in range(n_q):
        o.step(i)
        if i % 7 == 0 or i == n_q - 1:
            _check_query(i, o, out_a, sel_a, scores, w.k_blocks, True, stats)


def test_chunk_max_queries_sampled():
    """The largest chunk the call takes (QSA_MAX_CHUNK = 4096 tokens) at 20k
    context: 32 query groups of the score GEMM over its row ranges; every
    query's ids checked for validity, sampled queries against the oracle at
    their own position."""
    from sparse_attention_decode_cache_amd import qsa as Q
    n_q = Q.QSA_MAX_CHUNK
    w = with_size(W.CTX64K, n0=20003, steps=n_q)
    print(f"chunk {w.name}: n0={w.n0} n_q={n_q}", flush=True)
    g = GpuLayer(w)
    out, sel, scores = _chunk(g, n_q)
    assert np.isfinite(out).all()
    for i in range(n_q):
        nb = (w.n0 + i + 1) // 4
        row = sel[i]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < nb, f"query {i} ids"
    o = _Mirror(w)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in [0, 1, 127, 128, 1023, 2048, 3001, 4094, 4095]:
        pos = w.n0 + i
        if o.L.n < pos:
            rows = np.arange(o.L.n, pos)
            o.L.raw[rows] = W.host_raw_rows(w, rows, 0)
            o.L.K[rows], o.L.V[rows] = W.host_kv_rows(w, rows, 0)
            o.L.n = pos
        o.step(i)
        _check_query(i, o, out, sel, scores, w.k_blocks, True, stats)
    print(f"  {stats}")
