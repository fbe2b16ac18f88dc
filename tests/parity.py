"""Parity rules between the HIP path and the CPU oracle.

Tolerances: scores within 1e-3 relative, attention within 2e-3 absolute,
block ids bit-exact wherever the k-th / (k+1)-th score gap exceeds 1e-3
(relative), otherwise accepted by score threshold.  "Relative" for a score is
taken against A_b = sum_h |w_h| sum_i |q_hi * khat_bhi|, the scale of any
evaluation order's rounding error (A_b >= |s_b|), so that cancellation near 0
does not make a correct sum fail.

Summary rows have no stated tolerance; the one used here follows from the
arithmetic: both sides compute in double and round once to the storage type,
so they differ only when the two double results straddle a rounding boundary
-- at most one unit in the last place, and rarely.
"""
import numpy as np

SCORE_RTOL = 1e-3
ATTN_ATOL = 2e-3
TOPK_GAP = 1e-3


def f16_ulps(a, b):
    """|a - b| in binary16 units in the last place (a, b float16 arrays)."""
    def ordered(x):
        u = x.view(np.uint16).astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)   # -0 and +0 both 0x8000
    return np.abs(ordered(np.ascontiguousarray(a)) - ordered(np.ascontiguousarray(b)))


def f32_ulps(a, b):
    def ordered(x):
        u = np.ascontiguousarray(x).view(np.uint32).astype(np.int64)
        return np.where(u & 0x80000000, 0x80000000 - (u & 0x7FFFFFFF), 0x80000000 + u)
    return np.abs(ordered(a) - ordered(b))


def check_summaries(gpu, ref):
    """P1: <= 1 ulp everywhere; returns the count of differing elements."""
    assert gpu.shape == ref.shape and gpu.dtype == ref.dtype
    u = f16_ulps(gpu, ref) if gpu.dtype == np.float16 else f32_ulps(gpu, ref)
    assert int(u.max(initial=0)) <= 1, f"summary off by {int(u.max())} ulp"
    return int((u > 0).sum())


def check_scores(gpu, ref, scale):
    """P2: |s_gpu - s_ref| <= 1e-3 * A_b.  Returns max |err| / A_b."""
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = SCORE_RTOL * scale
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{bad.size} scores out of tolerance, first b={bad[0]}: {gpu[bad[0]]} vs {ref[bad[0]]}"
    return float(np.max(err / np.maximum(scale, 1e-300), initial=0.0))


def check_topk(sel, ref_scores, scale, k):
    """P3.  Returns 'exact' or 'threshold' (the branch the rule took)."""
    nb = ref_scores.shape[0]
    kb = min(k, nb)
    sel = np.asarray(sel, dtype=np.int64)
    assert sel.shape == (kb,), f"{sel.shape} ids, expected {kb}"
    if kb == 0:
        return "exact"
    assert np.all(np.diff(sel) > 0), "ids not strictly ascending"
    assert sel[0] >= 0 and sel[-1] < nb, "id out of range"
    if k >= nb:
        assert np.array_equal(sel, np.arange(nb))
        return "exact"
    order = np.lexsort((np.arange(nb), -ref_scores))
    sk, sk1 = ref_scores[order[kb - 1]], ref_scores[order[kb]]
    if sk - sk1 > TOPK_GAP * max(abs(sk), abs(sk1)):
        assert np.array_equal(sel, np.sort(order[:kb])), "top-k set differs from the oracle's"
        return "exact"
    chosen = np.zeros(nb, bool)
    chosen[sel] = True
    tol = TOPK_GAP * scale
    assert np.all(ref_scores[chosen] >= sk - tol[chosen]), "a chosen block scores below the k-th"
    assert np.all(ref_scores[~chosen] <= sk + tol[~chosen]), "an unchosen block scores above the k-th"
    return "threshold"


def check_topk_on_gpu_scores(sel, gpu_scores, k):
    """The GPU's chosen ids against the oracle's top-k rule applied to the
    GPU's own fp32 scores (the values its keys were made from): with equal
    scores on both sides the selection has one correct answer, so the ids
    must match bit for bit, whatever the gap at the k-th."""
    import oracle
    nb = int(np.asarray(gpu_scores).shape[0])
    ref = oracle.topk(np.asarray(gpu_scores, dtype=np.float32).astype(np.float64), k)
    sel = np.asarray(sel, dtype=np.int64)
    assert sel.shape == (min(k, nb),), f"{sel.shape} ids, expected {min(k, nb)}"
    bad = np.nonzero(sel != ref)[0]
    assert bad.size == 0, f"top-k differs from the rule on the GPU's scores at slot {bad[0]}: {sel[bad[0]]} vs {ref[bad[0]]}"


def check_attention(gpu, ref):
    """P4: <= 2e-3 absolute per element.  Returns the max error."""
    err = np.abs(gpu.astype(np.float64) - ref)
    m = float(err.max(initial=0.0))
    assert m <= ATTN_ATOL, f"attention max abs error {m}"
    return m
