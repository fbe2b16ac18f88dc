"""The planted workload against the oracle (CPU): the planted blocks take
the top ranks in the intended order, and the k-th / (k+1)-th gap is the
intended one, so that the top-k rule takes its exact branch."""
import dataclasses

import numpy as np

import oracle
import planted as PL
from parity import check_topk
from qsagen import workloads as W


def _scores(w, p, layer=0):
    nb = w.n0 // 4
    raw = W.host_raw_rows(w, np.arange(w.n0), layer)
    PL.apply_host(p, raw)
    gamma = W.host_gamma(w, layer)
    summ = oracle.full_summaries(raw, nb, gamma, w.rms_eps, w.rope_theta)
    s, scale = oracle.scores(summ, nb, p.q_idx, p.w, with_scale=True)
    return s, scale


def test_planted_ranks_and_gap():
    # the 64k layer shapes over 12,288 tokens: 3,072 blocks, 600 planted
    w = dataclasses.replace(W.CTX64K, n0=12288)
    p = PL.make(w, layer=0)
    s, scale = _scores(w, p)
    order = np.argsort(-s, kind="stable")
    k = w.k_blocks
    # the planted blocks are the top N_PLANT, ranked as planted
    top = order[:PL.N_PLANT]
    assert set(top.tolist()) == set(p.blocks.tolist())
    want = p.blocks[np.argsort(p.rank)]
    assert np.array_equal(top, want)
    gap = (s[order[k - 1]] - s[order[k]]) / s[order[k - 1]]
    assert abs(gap - PL.GAP) < 5e-4, gap
    # far above every random block
    assert s[order[PL.N_PLANT - 1]] > 1.2 * s[order[PL.N_PLANT]]
    assert check_topk(np.sort(order[:k]), s, scale, k) == "exact"


def test_targets_shape():
    t = PL.targets(512)
    assert np.all(np.diff(t) < 0)
    assert abs(t[511] / t[512] - (1 + PL.GAP)) < 1e-12
    assert abs(t[511] - PL.T_K) < 1e-12
