"""The ablations (the page's own comparisons, as library calls) against the
path they stand beside and against the CPU oracle.

- pooled-key cache off (qsa_state_invalidate(st, 0) before every step): every
  block pooled again each step; results bitwise equal to the cache-on run;
- cell-level top-k (qsa_topk_cells): block scores expanded to cells, then a
  top-k over cells; the cells of the blocks the block-level top-k chooses,
  plus the tail;
- gather off (qsa_attend_masked): flash-decode over every cached row with the
  unselected blocks masked; the gathered attention's result."""
import numpy as np
import pytest

import oracle
from parity import check_attention, check_topk
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def test_cache_off_is_bitwise_the_cache_on_step():
    """Two copies of one layer: one keeps its pooled cache, the other pools
    every block again before each step; outputs, ids and scores are equal bit
    for bit (the same pooling routine writes the same rows)."""
    w = with_size(W.CTX64K, n0=9001, steps=6)
    a, b = GpuLayer(w), GpuLayer(w)
    for s in range(w.steps):
        ra = a.step(s)
        b.qsa.qsa_state_invalidate(b.state, 0)
        rb = b.step(s)
        assert np.array_equal(ra["out"], rb["out"]), f"step {s}: outputs differ"
        assert np.array_equal(ra["sel"], rb["sel"]) and np.array_equal(ra["scores"], rb["scores"])
    nb = a.state.n_tokens // 4
    assert np.array_equal(a.buf.summary[:nb].cpu().numpy(), b.buf.summary[:nb].cpu().numpy())


def _cells_vs_blocks(scores, n, top_k, qsa):
    import torch
    nb = n // 4
    ws = qsa.ablation_workspace(qsa.make_desc(4, 128, qsa.QSA_F16, 16, 2, 256, top_k),
                                (n + 3) // 4 * 4)
    tail = n % 4
    kept = min(top_k, 4 * nb)
    cells = torch.full((kept + tail + 8,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_topk_cells(scores, n, top_k, cells, ws)
    sel = torch.full((max(min(top_k // 4, nb), 1),), -7, dtype=torch.int32, device="cuda")
    if nb > 0:
        qsa.qsa_topk_blocks(scores, nb, top_k // 4, sel, ws)
    torch.cuda.synchronize()
    c = cells.cpu().numpy()
    assert np.all(c[kept + tail:] == -7), "written past the cells"
    want = oracle.cells(sel.cpu().numpy()[:min(top_k // 4, nb)], n)
    assert np.array_equal(c[:kept + tail], want)
    return c[:kept + tail]


@pytest.mark.parametrize("n", [61789, 61790, 61791, 61792, 2040, 2049, 3])
def test_topk_cells_is_the_block_topk_expanded(n):
    """Random fp32 scores: the cell-level top-k picks the cells of the blocks
    the block-level top-k picks (every tail length; fewer cells than k)."""
    import torch
    import sparse_attention_decode_cache_amd as qsa
    g = torch.Generator().manual_seed(n)
    scores = torch.randn(max(n // 4, 1), generator=g).cuda()
    _cells_vs_blocks(scores, n, 2048, qsa)


def test_topk_cells_with_tied_block_scores():
    """Scores on a coarse grid (many equal blocks across the k-th): cell
    order breaks ties by cell, which is block order, so the chosen cells are
    still whole blocks, the same as the block top-k's."""
    import torch
    import sparse_attention_decode_cache_amd as qsa
    g = torch.Generator().manual_seed(11)
    scores = torch.randint(0, 40, (30000,), generator=g).float().cuda()
    c = _cells_vs_blocks(scores, 4 * 30000 + 2, 2048, qsa)
    assert np.all(np.bincount(c[:-2] // 4) % 4 == 0)


def test_topk_cells_decode_step_scores_against_oracle():
    """The decode step's own scores at 64k: the cells' blocks satisfy the
    top-k rule against the oracle's scores."""
    import torch
    w = with_size(W.CTX64K, n0=61789, steps=1)
    g = GpuLayer(w)
    o = OracleMirror(w)
    rg = g.step(0)
    ro = o.step(0)
    n = rg["n"]
    scores = torch.from_numpy(rg["scores"]).cuda()
    c = _cells_vs_blocks(scores, n, w.top_k_tokens, g.qsa)
    blocks = np.unique(c[c < 4 * (n // 4)] // 4)
    check_topk(blocks, ro["scores"], ro["scale"], w.k_blocks)


def _masked_case(base, n0, steps=2, sel_override=None):
    import torch
    w = with_size(base, n0=n0, steps=steps)
    print(f"masked {w.name}: n0={n0} Hq={w.q_heads} Hkv={w.kv_heads} Dh={w.head_dim}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    ws = g.qsa.ablation_workspace(g.desc, g.cap)
    worst = 0.0
    for s in range(steps):
        rg = g.step(s)
        o.step(s)
        n = rg["n"]
        sel = rg["sel"] if sel_override is None else sel_override(n)
        dsel = torch.zeros(max(len(sel), 1), dtype=torch.int32, device="cuda")   # never NULL
        dsel[:len(sel)] = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
        q = g.inp.q[s]
        masked = torch.full((w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        gathered = torch.full_like(masked, float("nan"))
        g.qsa.qsa_attend_masked(g.desc, g.buf.cache, n, dsel, len(sel), q, masked, ws)
        g.qsa.qsa_gather_attend(g.desc, g.buf.cache, n, dsel, len(sel), q, gathered, g.ws)
        torch.cuda.synchronize()
        mk = masked.cpu().numpy().astype(np.float64)
        ga = gathered.cpu().numpy().astype(np.float64)
        ref = oracle.attend(q.cpu().numpy(), o.L.K, o.L.V, oracle.cells(sel, n))
        worst = max(worst, check_attention(mk, ref))
        assert np.max(np.abs(mk - ga)) <= 1e-4, "masked and gathered attention differ"
    print(f"  max |err| {worst:.2e}")


def test_attend_masked_headline_shapes():
    """16 q / 2 KV heads x 256, K = 512 blocks, every tail length."""
    _masked_case(W.CTX64K, 12001, steps=4)


@pytest.mark.parametrize("q_heads,kv_heads,head_dim", [(2, 2, 128), (8, 2, 64), (4, 4, 256), (8, 1, 128)])
def test_attend_masked_shapes(q_heads, kv_heads, head_dim):
    base = with_size(W.CTX64K, q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim)
    _masked_case(base, 5003, steps=1)


def test_attend_masked_sparse_and_empty_selections():
    """A handful of blocks, and none at all (only the tail takes part)."""
    _masked_case(W.CTX64K, 4001, steps=1, sel_override=lambda n: np.array([0, 7, 500, n // 4 - 1]))
    _masked_case(W.TINY, 4097, steps=1, sel_override=lambda n: np.zeros(0, np.int32))


def test_attend_masked_256k():
    """Every cached row at 255,182 tokens read, the decode step's selection
    applied as the mask."""
    _masked_case(W.CTX256K, 255181, steps=1)
