"""Batched variable-length decode (qsa_decode_step_batch) against the CPU
oracle, sequence by sequence: each sequence of the batch must give what its
own decode step gives.  The sequences share the layer (its shapes and gamma)
and nothing else: own caches, contexts, positions and queries."""
import numpy as np
import pytest

import oracle
from parity import check_attention, check_summaries, check_topk, check_topk_on_gpu_scores
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _batch_io(g, s, sel):
    inp = g.inp
    return {"idx_k_row": inp.raw[s], "k_row": inp.k[s], "v_row": inp.v[s], "q_idx": inp.q_idx[s],
            "w": inp.w[s], "q": inp.q[s], "out": g.out, "sel_out": sel, "scores_out": g.scores}


def _run_batch(base, contexts, steps, check_sel=True):
    import torch
    import sparse_attention_decode_cache_amd as qsa
    print(f"batch {base.name}: contexts {contexts}, steps {steps}, K={base.k_blocks}", flush=True)
    ws_ = [with_size(base, n0=n0, steps=steps) for n0 in contexts]
    gs = [GpuLayer(w, seq=i, gamma_seq=0) for i, w in enumerate(ws_)]
    os_ = [OracleMirror(w, seq=i, gamma_seq=0) for i, w in enumerate(ws_)]
    desc = gs[0].desc
    ws = qsa.batch_workspace(desc, [g.cap for g in gs])
    sels = [torch.full((base.k_blocks,), -1, dtype=torch.int32, device="cuda") for _ in gs]
    stats = {"exact": 0, "threshold": 0, "attn_err": 0.0, "ulp_diffs": 0}
    for s in range(steps):
        qsa.qsa_decode_step_batch(desc, [g.buf.cache for g in gs], [g.state for g in gs],
                                  [_batch_io(g, s, sels[i]) for i, g in enumerate(gs)],
                                  gs[0].gamma, ws)
        for i, (g, o) in enumerate(zip(gs, os_)):
            ro = o.step(s)
            n = g.state.n_tokens
            nb = n // 4
            assert n == o.L.n, (i, n, o.L.n)
            summ = g.buf.summary[:nb].cpu().numpy()
            stats["ulp_diffs"] += check_summaries(summ, o.L.summary[:nb])
            sel = sels[i][:min(base.k_blocks, nb)].cpu().numpy()
            out = g.out.cpu().numpy().astype(np.float64)
            branch = check_topk(sel, ro["scores"], ro["scale"], base.k_blocks)
            stats[branch] += 1
            if nb > 0:
                check_topk_on_gpu_scores(sel, g.scores[:nb].cpu().numpy(), base.k_blocks)
            cells = oracle.cells(sel, n)
            assert len(cells) == oracle.n_cells(n, base.k_blocks)
            ref = oracle.attend(ro["q"], o.L.K, o.L.V, cells)
            stats["attn_err"] = max(stats["attn_err"], check_attention(out, ref))
            if branch == "exact":
                check_attention(out, ro["out"])
    print(f"  {stats}")
    return stats


def test_batch_gqa_mixed_contexts():
    """4 x 128 f16 indexer, 16/2 x 256 attention, top-k 2048 tokens: one sequence
    that keeps every block, three that select, positions crossing block ends."""
    st = _run_batch(W.CTX64K, [1201, 2047, 4099, 9001], steps=6)
    assert st["exact"] + st["threshold"] == 24


def test_batch_tiny_eight_sequences():
    """The 1 x 64 fp32 indexer, 4/1 x 64 attention shape, 8 sequences (the
    maximum), contexts from empty to past the top-k."""
    w = with_size(W.TINY, top_k_tokens=64)
    _run_batch(w, [0, 3, 17, 64, 255, 256, 1001, 4096], steps=9)


def test_batch_single_sequence_matches_decode_step():
    """A batch of one agrees with qsa_decode_step on the same inputs whenever
    both keep every block: the same summary bits (the same pooling), and the
    same attention up to summation order (the batch attends in 64-cell
    iterations, the single step in 16-cell splits) -- far inside 2e-3."""
    import torch
    import sparse_attention_decode_cache_amd as qsa
    w = with_size(W.TINY, n0=40, steps=4, top_k_tokens=256)
    a, b = GpuLayer(w, seq=3), GpuLayer(w, seq=3)
    ws = qsa.batch_workspace(a.desc, [a.cap])
    for s in range(4):
        qsa.qsa_decode_step_batch(a.desc, [a.buf.cache], [a.state], [_batch_io(a, s, None)], a.gamma, ws)
        b.step(s)
        nb = a.state.n_tokens // 4
        assert a.state.n_tokens == b.state.n_tokens
        torch.testing.assert_close(a.out, b.out, rtol=0.0, atol=1e-5)
        assert torch.equal(a.buf.summary[:nb], b.buf.summary[:nb])


def test_batch_full_size_mixed_contexts():
    """The benchmarked batch (8 sequences of 16,381 .. 255,181 tokens, the
    headline layer shapes): tile lists of 32, 16 and 8 entries side by side in
    one select launch; every sequence checked against its own oracle."""
    st = _run_batch(W.BATCH, list(W.BATCH_CONTEXTS), steps=2)
    assert st["exact"] + st["threshold"] == 16


def test_batch_winners_clustered_in_a_few_tiles():
    """The batched select with every winner of two sequences inside a few
    consecutive tiles (tile lists of 16 and 32 entries): the per-sequence
    fallback over every key, beside a sequence the lists decide."""
    import torch
    import sparse_attention_decode_cache_amd as qsa
    contexts, clusters = [61789, 29453, 126253], [(3000, 3700), (100, 900), None]
    ws_ = [with_size(W.CTX64K, n0=n0, steps=1) for n0 in contexts]
    gs = [GpuLayer(w, seq=i, gamma_seq=0) for i, w in enumerate(ws_)]
    os_ = [OracleMirror(w, seq=i, gamma_seq=0) for i, w in enumerate(ws_)]
    for w, g, o, cl in zip(ws_, gs, os_, clusters):
        if cl:
            qi, _, _ = W.host_step_inputs(w, 0, 0, o.seq)
            rows = np.stack([(qi * (4.0 + 0.01 * (b - cl[0]))).astype(np.float16)
                             for b in range(*cl)])
            o.L.summary[cl[0]:cl[1]] = rows
            g.buf.summary[cl[0]:cl[1]] = torch.from_numpy(rows).cuda()
    desc = gs[0].desc
    ws = qsa.batch_workspace(desc, [g.cap for g in gs])
    sels = [torch.full((W.CTX64K.k_blocks,), -1, dtype=torch.int32, device="cuda") for _ in gs]
    qsa.qsa_decode_step_batch(desc, [g.buf.cache for g in gs], [g.state for g in gs],
                              [_batch_io(g, 0, sels[i]) for i, g in enumerate(gs)], gs[0].gamma, ws)
    for i, (g, o, cl) in enumerate(zip(gs, os_, clusters)):
        ro = o.step(0)
        n = g.state.n_tokens
        sel = sels[i].cpu().numpy()
        branch = check_topk(sel, ro["scores"], ro["scale"], W.CTX64K.k_blocks)
        check_topk_on_gpu_scores(sel, g.scores[:n // 4].cpu().numpy(), W.CTX64K.k_blocks)
        if cl:
            assert branch == "exact" and np.array_equal(sel, np.arange(cl[1] - 512, cl[1]))
        ref = oracle.attend(ro["q"], o.L.K, o.L.V, oracle.cells(sel, n))
        check_attention(g.out.cpu().numpy().astype(np.float64), ref)
