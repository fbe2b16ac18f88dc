"""The top-k's exact branch on the histogram fast path: the planted
workload (tests/planted.py) at the 64k, 128k and 256k layer shapes and real
context lengths.  Every step's ids must equal the oracle's bit for bit (the
k-th / (k+1)-th gap is 3e-3, above the rule's 1e-3), and once the window has
followed the planted scores (the first steps may take the full top-k) the
step must take the histogram path."""
import pytest

import planted as PL
from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W
from test_gpu_decode import _compare_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [W.CTX64K, W.CTX128K, W.CTX256K], ids=lambda w: w.name)
def test_planted_exact_branch_on_fast_path(w):
    w = with_size(w, steps=8)
    print(f"planted decode {w.name} n0={w.n0}", flush=True)
    p = PL.make(w, layer=0)
    g = GpuLayer(w, planted=p)
    o = OracleMirror(w, planted=p)
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    paths = []
    for s in range(w.steps):
        _compare_step(g, o, s, stats)
        paths.append(g.path())
    print(f"  {stats} paths {paths}")
    assert stats["exact"] == w.steps, stats
    assert all(x == g.qsa.QSA_PATH_HIST for x in paths[2:]), paths
