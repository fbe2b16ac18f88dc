"""Multi-query decode (qsa_decode_step_multi) against the CPU oracle.

Token i of a call must give what the i-th of as many decode steps in a row
gives: its scores over the blocks completed by then (a causal block mask),
its top-k and its attention.  The speculative-verify flow -- draft tokens
decoded together, the rejected ones dropped with qsa_state_truncate -- must
leave a cache whose next steps match an oracle that saw the same appends and
the same truncation (dirty-range protection: a block that held a dropped
token is pooled again once it is completed by the tokens that replace it).

Inputs are the seeded host streams; rejected drafts take their rows from a
different stream than the tokens that replace them."""
import numpy as np
import pytest

import oracle
from parity import check_attention, check_scores, check_summaries, check_topk, check_topk_on_gpu_scores
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu

DRAFT_SEQ = 7      # stream id of the rows and queries of rejected drafts


def _host_tokens(w, positions, row_seqs, steps):
    """Rows at `positions` (stream row_seqs[i]) and the queries of `steps`."""
    raw, k, v, qi, wt, q = [], [], [], [], [], []
    for pos, rs, st in zip(positions, row_seqs, steps):
        raw.append(W.host_raw_rows(w, [pos], 0, rs)[0])
        kk, vv = W.host_kv_rows(w, [pos], 0, rs)
        k.append(kk[0])
        v.append(vv[0])
        a, b, c = W.host_step_inputs(w, 0, st, rs)
        qi.append(a)
        wt.append(b)
        q.append(c)
    return [np.ascontiguousarray(np.stack(x)) for x in (raw, k, v, qi, wt, q)]


def _multi(g, toks):
    """One qsa_decode_step_multi call on g with host inputs `toks`."""
    import torch
    raw, k, v, qi, wt, q = (torch.from_numpy(x).cuda() for x in toks)
    n_q = raw.shape[0]
    n0 = g.state.n_tokens
    nb_last = (n0 + n_q) // 4
    w = g.w
    ws = g.qsa.multi_workspace(g.desc, g.cap, n_q)
    out = torch.full((n_q, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((n_q, w.k_blocks), -7, dtype=torch.int32, device="cuda")
    scores = torch.full((n_q, max(nb_last, 1)), float("nan"), dtype=torch.float32, device="cuda")
    g.qsa.qsa_decode_step_multi(g.desc, g.buf.cache, g.state, n_q, raw, k, v, g.gamma, qi, wt, q,
                                out, sel, scores, ws)
    torch.cuda.synchronize()
    assert (g.state.n_tokens, g.state.n_valid_blocks) == (n0 + n_q, nb_last)
    return out.cpu().numpy().astype(np.float64), sel.cpu().numpy(), scores.cpu().numpy(), nb_last


def _check(i, L, toks, res, k_blocks, stats):
    """Query i of a call against the oracle layer L, which has just taken it."""
    out, sel, scores, nb_last = res
    raw, kr, vr, qi, wt, q = toks
    n = L.n
    nb = n // 4
    kb = min(k_blocks, nb)
    s_ref, scale = oracle.scores(L.summary, nb, qi[i], wt[i], with_scale=True)
    assert np.all(sel[i, kb:] == -1), f"query {i}: slots past {kb} not -1"
    if nb > 0:
        check_scores(scores[i, :nb], s_ref, scale)
    if nb_last > 0:
        assert np.all(scores[i, nb:nb_last] == -np.inf), f"query {i}: masked scores not -inf"
    branch = check_topk(sel[i, :kb], s_ref, scale, k_blocks)
    stats[branch] += 1
    if nb > 0:
        check_topk_on_gpu_scores(sel[i, :kb], scores[i, :nb], k_blocks)
    cells = oracle.cells(sel[i, :kb], n)
    assert len(cells) == oracle.n_cells(n, k_blocks)
    ref = oracle.attend(q[i], L.K, L.V, cells)
    stats["attn_err"] = max(stats["attn_err"], check_attention(out[i], ref))
    if branch == "exact":
        exact = oracle.attend(q[i], L.K, L.V, oracle.cells(oracle.topk(s_ref, k_blocks), n))
        check_attention(out[i], exact)


def _oracle_take(L, toks, i):
    raw, kr, vr, qi, wt, q = toks
    L.append(raw[i], kr[i], vr[i])
    L.rebuild()


def _run(base, n0, n_q, calls=1):
    """`calls` multi-query calls of n_q true tokens each, every query checked."""
    w = with_size(base, n0=n0, steps=n_q * calls)
    print(f"multi {w.name}: n0={n0} n_q={n_q} calls={calls} K={w.k_blocks}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for c in range(calls):
        p = g.state.n_tokens
        steps = list(range(p - n0, p - n0 + n_q))
        toks = _host_tokens(w, range(p, p + n_q), [0] * n_q, steps)
        res = _multi(g, toks)
        for i in range(n_q):
            _oracle_take(o.L, toks, i)
            _check(i, o.L, toks, res, w.k_blocks, stats)
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])
    print(f"  {stats}")
    return stats


@pytest.mark.parametrize("n0", [3000, 3001, 3002, 3003])
@pytest.mark.parametrize("n_q", [2, 3, 4])
def test_multi_every_alignment(n0, n_q):
    """4 x 128 f16 indexer, 16/2 x 256 attention, K = 512 blocks; every
    alignment of the first token to the 4-token block, so the block the call
    completes falls on each query in turn."""
    st = _run(W.CTX64K, n0, n_q, calls=3)
    assert st["exact"] + st["threshold"] == 3 * n_q


def test_multi_fp32_indexer_tiny():
    """1 x 64 fp32 indexer, 4/1 x 64 attention, K = 64 blocks."""
    st = _run(W.TINY, 4094, 4, calls=4)
    assert st["exact"] + st["threshold"] == 16


def test_multi_from_empty_cache():
    """From position 0 with K = 4 blocks: tail-only queries, keep-every-block
    queries, then selecting queries."""
    w = with_size(W.TINY, top_k_tokens=16)
    st = _run(w, 0, 3, calls=9)
    assert st["exact"] == 27


def test_multi_crosses_top_k():
    """Queries of one call on both sides of K: the first keeps every block,
    the last selects."""
    st = _run(W.CTX64K, 2047, 4, calls=2)
    assert st["exact"] + st["threshold"] == 8


def test_multi_single_query_is_a_decode_step():
    st = _run(W.CTX64K, 5001, 1, calls=3)
    assert st["exact"] + st["threshold"] == 3


@pytest.mark.parametrize("idx_heads,idx_dim,idx_f16", [(1, 128, True), (4, 64, False), (1, 64, True)])
def test_multi_indexer_shapes(idx_heads, idx_dim, idx_f16):
    base = with_size(W.CTX64K, idx_heads=idx_heads, idx_dim=idx_dim, idx_f16=idx_f16)
    st = _run(base, 4001, 3, calls=2)
    assert st["exact"] + st["threshold"] == 6


@pytest.mark.parametrize("q_heads,kv_heads,head_dim", [(2, 2, 128), (8, 2, 64), (4, 4, 256)])
def test_multi_attention_shapes(q_heads, kv_heads, head_dim):
    base = with_size(W.CTX64K, q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim)
    st = _run(base, 3001, 4, calls=2)
    assert st["exact"] + st["threshold"] == 8


def test_speculative_verify_flow():
    """Rounds of verify calls with 1 + 3 drafts: a tokens accepted, the rest
    rejected and dropped with qsa_state_truncate; the next call re-appends
    at the first dropped position with the true rows.  Every query of every
    call is checked (the oracle takes the same appends and truncations), then
    the pooled cache and one plain decode step after the last round."""
    import torch
    w = with_size(W.CTX64K, n0=3001, steps=64)
    g = GpuLayer(w)
    o = OracleMirror(w)
    accepts = [0, 4, 1, 2, 3, 0, 2, 4, 1, 3, 2, 1]    # accepted tokens of each call
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    step = 0
    for a in accepts:
        p = g.state.n_tokens
        assert p == o.L.n
        seqs = [0] * a + [DRAFT_SEQ] * (4 - a)
        toks = _host_tokens(w, range(p, p + 4), seqs, range(step, step + 4))
        res = _multi(g, toks)
        for i in range(4):
            _oracle_take(o.L, toks, i)
            _check(i, o.L, toks, res, w.k_blocks, stats)
        print(f"  call at {p}: accepted {a}, watermark {g.state.n_valid_blocks}", flush=True)
        g.qsa.qsa_state_truncate(g.state, p + a)
        o.L.truncate(p + a)
        assert (g.state.n_tokens, g.state.n_valid_blocks) == (o.L.n, o.L.valid)
        step += a
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])
    # a plain decode step at the end pools any dirty block again
    for extra in range(4):
        p = g.state.n_tokens
        toks = _host_tokens(w, [p], [0], [step])
        raw, kr, vr, qi, wt, q = (torch.from_numpy(x).cuda() for x in toks)
        g.qsa.qsa_decode_step(g.desc, g.buf.cache, g.state, raw[0], kr[0], vr[0], g.gamma, qi[0],
                              wt[0], q[0], g.out, g.sel, g.scores, g.ws)
        torch.cuda.synchronize()
        _oracle_take(o.L, toks, 0)
        out = g.out.cpu().numpy().astype(np.float64)[None]
        nbx = g.state.n_tokens // 4
        kb = min(w.k_blocks, nbx)
        sel = np.full((1, w.k_blocks), -1, np.int32)
        sel[0, :kb] = g.sel[:kb].cpu().numpy()
        sc = g.scores[:nbx].cpu().numpy()[None]
        _check(0, o.L, toks, (out, sel, sc, nbx), w.k_blocks, stats)
        step += 1
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])
    print(f"  {stats}")


def test_multi_256k_four_queries():
    """The 256k layer shapes at 255,181 tokens: four queries in one call,
    each against the oracle at its own position."""
    w = with_size(W.CTX256K, n0=255181, steps=4)
    print(f"multi {w.name}: n0={w.n0} n_q=4", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    toks = _host_tokens(w, range(w.n0, w.n0 + 4), [0] * 4, range(4))
    res = _multi(g, toks)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in range(4):
        _oracle_take(o.L, toks, i)
        _check(i, o.L, toks, res, w.k_blocks, stats)
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[nb - 64:nb].cpu().numpy(), o.L.summary[nb - 64:nb])
    print(f"  {stats}")


def test_multi_argument_errors():
    import torch
    w = with_size(W.TINY, n0=100, steps=8)
    g = GpuLayer(w)
    toks = [torch.from_numpy(x).cuda() for x in _host_tokens(w, range(100, 105), [0] * 5, range(5))]
    raw, k, v, qi, wt, q = toks
    ws = g.qsa.multi_workspace(g.desc, g.cap, 4)
    out = torch.empty((5, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(g.qsa.QSAError):      # n_q above the maximum
        g.qsa.qsa_decode_step_multi(g.desc, g.buf.cache, g.state, 5, raw, k, v, g.gamma, qi, wt, q,
                                    out, None, None, ws)
    with pytest.raises(g.qsa.QSAError):      # workspace for 2 queries, 4 asked
        small = g.qsa.multi_workspace(g.desc, g.cap, 2)
        g.qsa.qsa_decode_step_multi(g.desc, g.buf.cache, g.state, 4, raw, k, v, g.gamma, qi, wt, q,
                                    out, None, None, small)
    g.state.n_tokens = g.cap - 2
    with pytest.raises(g.qsa.QSAError):      # past the capacity
        g.qsa.qsa_decode_step_multi(g.desc, g.buf.cache, g.state, 3, raw, k, v, g.gamma, qi, wt, q,
                                    out, None, None, ws)
    assert g.state.n_tokens == g.cap - 2


def test_multi_after_invalidation_rebuilds():
    """The watermark far below the call (a state load): the call appends its
    rows and rebuilds every distrusted block in its own launch before the one
    pass over the summaries."""
    w = with_size(W.CTX64K, n0=5002, steps=4)
    g = GpuLayer(w)
    o = OracleMirror(w)
    g.qsa.qsa_state_invalidate(g.state, 1003)
    o.L.invalidate(1003)
    toks = _host_tokens(w, range(w.n0, w.n0 + 4), [0] * 4, range(4))
    res = _multi(g, toks)
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0}
    for i in range(4):
        _oracle_take(o.L, toks, i)
        _check(i, o.L, toks, res, w.k_blocks, stats)
    nb = g.state.n_valid_blocks
    check_summaries(g.buf.summary[:nb].cpu().numpy(), o.L.summary[:nb])
    assert stats["exact"] + stats["threshold"] == 4
