"""The fused decode step against the CPU oracle, step by step."""
import numpy as np
import pytest

import oracle
from parity import check_attention, check_scores, check_summaries, check_topk, check_topk_on_gpu_scores
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _compare_step(g, o, s, stats):
    rg = g.step(s)
    ro = o.step(s)
    n, nb = rg["n"], rg["nb"]
    assert n == o.L.n
    summ = g.buf.summary[:nb].cpu().numpy()
    stats["ulp_diffs"] += check_summaries(summ, o.L.summary[:nb])
    if nb > 0:
        check_scores(rg["scores"], ro["scores"], ro["scale"])
    branch = check_topk(rg["sel"], ro["scores"], ro["scale"], g.w.k_blocks)
    stats[branch] += 1
    if nb > 0:
        check_topk_on_gpu_scores(rg["sel"], rg["scores"], g.w.k_blocks)
    cells = oracle.cells(rg["sel"], n)
    assert len(cells) == oracle.n_cells(n, g.w.k_blocks) <= g.w.top_k_tokens + 3
    ref = oracle.attend(ro["q"], o.L.K, o.L.V, cells)
    stats["attn_err"] = max(stats["attn_err"], check_attention(rg["out"], ref))
    if branch == "exact":
        check_attention(rg["out"], ro["out"])
    return rg, ro


def _run(w, steps):
    print(f"decode {w.name} n0={w.n0} steps={steps} K={w.k_blocks}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    for s in range(steps):
        _compare_step(g, o, s, stats)
    print(f"  {stats}")
    return g, o, stats


def test_decode_tiny_every_step():
    """4096-token context, 1 x 64 fp32 indexer, 4/1 x 64 attention, top-k 256 tokens, 32 steps."""
    _run(W.TINY, W.TINY.steps)


def test_decode_from_empty_cache():
    """n = 1, 2, ...: tail-only steps, every-block steps, then real selection (K = 4 blocks)."""
    w = with_size(W.TINY, n0=0, steps=48, top_k_tokens=16)
    _, _, st = _run(w, w.steps)
    assert st["exact"] + st["threshold"] == 48


def test_decode_gqa_shape_16k():
    """The 64k/128k/256k layer shapes (4 x 128 f16 indexer, 16/2 x 256) at 16k context."""
    w = with_size(W.CTX64K, n0=16381, steps=12)
    _run(w, w.steps)


def test_invalidate_and_truncate_on_gpu():
    import torch
    import sparse_attention_decode_cache_amd as qsa
    w = with_size(W.TINY, n0=1500, steps=40, top_k_tokens=64)
    g = GpuLayer(w)
    o = OracleMirror(w)
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    for s in range(10):
        _compare_step(g, o, s, stats)
    # state load: distrust rows from position 777 on, poison them, continue
    qsa.qsa_state_invalidate(g.state, 777)
    assert g.state.n_valid_blocks == 777 // 4
    g.buf.summary[777 // 4:] = float("nan")
    for s in range(10, 20):
        _compare_step(g, o, s, stats)
    # sequence edit: drop the last 7 tokens on both sides, then append fresh rows
    pos = g.state.n_tokens - 7
    qsa.qsa_state_truncate(g.state, pos)
    o.L.truncate(pos)
    assert (g.state.n_tokens, g.state.n_valid_blocks) == (pos, min(pos // 4, o.L.valid)) == (o.L.n, o.L.valid)
    rng = np.random.default_rng(4)
    for s in range(12):
        raw = rng.normal(0, 1, w.idx_row).astype(np.float32)
        kr = rng.normal(0, 1, w.kv_row).astype(np.float16)
        vr = rng.normal(0, 1, w.kv_row).astype(np.float16)
        qi = rng.normal(0, 1, w.idx_row).astype(np.float32)
        wt = rng.uniform(0, 1, w.idx_heads).astype(np.float32)
        q = rng.normal(0, 1, (w.q_heads, w.head_dim)).astype(np.float32)
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        qsa.qsa_decode_step(g.desc, g.buf.cache, g.state, d(raw), d(kr), d(vr), g.gamma, d(qi), d(wt), d(q),
                            g.out, g.sel, g.scores, g.ws)
        r = o.L.step(raw, kr, vr, qi, wt, q)
        n = g.state.n_tokens
        nb = n // 4
        assert n == o.L.n
        summ = g.buf.summary[:nb].cpu().numpy()
        check_summaries(summ, o.L.summary[:nb])
        sc = oracle.scores(o.L.summary, nb, qi, wt, with_scale=True)[1]
        sel = g.sel[:min(w.k_blocks, nb)].cpu().numpy()
        check_topk(sel, r["scores"], sc, w.k_blocks)
        check_topk_on_gpu_scores(sel, g.scores[:nb].cpu().numpy(), w.k_blocks)
        check_attention(g.out.cpu().numpy(), oracle.attend(q, o.L.K, o.L.V, oracle.cells(sel, n)))


def test_decode_is_bitwise_repeatable():
    w = with_size(W.CTX64K, n0=9000, steps=2)
    a = GpuLayer(w)
    b = GpuLayer(w)
    for s in range(2):
        ra, rb = a.step(s), b.step(s)
        assert np.array_equal(ra["out"], rb["out"]) and np.array_equal(ra["sel"], rb["sel"])
        assert np.array_equal(ra["scores"], rb["scores"])


def _cluster_rows(w, lo, hi):
    """Summary rows for blocks [lo, hi) that outscore every other block for the
    step-0 query, increasing with the block id (no ties): f16 copies of
    q_idx scaled by 4 + 0.01 (b - lo)."""
    qi, _, _ = W.host_step_inputs(w, 0, 0)
    dt = np.float16 if w.idx_f16 else np.float32
    return np.stack([(qi * (4.0 + 0.01 * (b - lo))).astype(dt) for b in range(lo, hi)])


@pytest.mark.parametrize("n0,lo,hi", [(61789, 3000, 3700), (29453, 100, 900), (255181, 40000, 40600)])
def test_decode_winners_clustered_in_a_few_tiles(n0, lo, hi):
    """Every winner inside a few consecutive tiles, so those tiles' lists are
    full with their last entries above the k-th: the list fast path cannot
    decide and the top-k runs over every key (tile lists of 16, 32 and 8
    entries at these contexts).  The cluster's summary rows are written into
    the GPU cache and the oracle's alike."""
    import torch
    w = with_size(W.CTX64K, n0=n0, steps=1)
    g = GpuLayer(w)
    o = OracleMirror(w)
    rows = _cluster_rows(w, lo, hi)
    o.L.summary[lo:hi] = rows
    g.buf.summary[lo:hi] = torch.from_numpy(rows).cuda()
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    rg, ro = _compare_step(g, o, 0, stats)
    assert stats["exact"] == 1
    assert np.array_equal(rg["sel"], np.arange(hi - w.k_blocks, hi))


def test_decode_score_stage_alone():
    """qsa_decode_score runs the step's score pass alone: its scores equal
    qsa_index_score's bit for bit (same kernel arithmetic) and the oracle's to
    the score tolerance; the histogram it leaves makes the next step take the
    full top-k once, with the same results."""
    import numpy as np
    import torch
    import oracle
    from parity import check_scores
    w = with_size(W.CTX64K, steps=3)
    print(f"decode score stage {w.name} n0={w.n0}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    q = g.qsa
    nb = w.n0 // 4
    s1 = torch.empty(nb, dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    q.qsa_decode_score(g.desc, g.buf.cache, g.state, g.gamma, g.inp.q_idx[0], g.inp.w[0], s1, g.ws)
    q.qsa_index_score(g.desc, g.buf.cache, nb, g.inp.q_idx[0], g.inp.w[0], s2)
    assert g.state.n_tokens == w.n0
    a, b = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    q_idx, wt, _ = W.host_step_inputs(w, 0, 0)
    ref, scale = oracle.scores(o.L.summary, nb, q_idx, wt, with_scale=True)
    check_scores(a, ref, scale)
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    paths = []
    for s in range(w.steps):
        _compare_step(g, o, s, stats)
        paths.append(g.path())
    print(f"  {stats} paths {paths}")
    assert paths[0] == q.QSA_PATH_FULL and all(p == q.QSA_PATH_HIST for p in paths[1:]), paths
