"""Full-size parity: the 64k, 128k and 256k layer shapes at their real context
lengths, and the same shapes at 300,000 and 524,000 tokens (past the 65,536
blocks an earlier top-k held in one workgroup's bitmap), driven through the
same decode-step call and launch configuration the benchmark times.  The oracle regenerates every input on the host (seeded
generator) and recomputes the whole path in double for each step: every
summary row, every score, the top-k rule and the attention output are checked.
"""
import pytest

from gpu_layer import GpuLayer, OracleMirror, with_size
from qsagen import workloads as W
from test_gpu_decode import _compare_step

pytestmark = pytest.mark.gpu


CTX300K = with_size(W.CTX256K, n0=300000, name="qsa-300k")
CTX524K = with_size(W.CTX256K, n0=524000, name="qsa-524k")


@pytest.mark.parametrize("w", [W.CTX64K, W.CTX128K, W.CTX256K, CTX300K, CTX524K], ids=lambda w: w.name)
def test_fullsize_decode_parity(w):
    w = with_size(w, steps=8)            # 8 steps: two block completions
    print(f"fullsize decode {w.name} n0={w.n0}", flush=True)
    g = GpuLayer(w)
    o = OracleMirror(w)
    stats = {"ulp_diffs": 0, "exact": 0, "threshold": 0, "attn_err": 0.0}
    paths = []
    for s in range(w.steps):
        _compare_step(g, o, s, stats)
        paths.append(g.path())
    print(f"  {stats} paths {paths}")
    # the first step on a fresh workspace may not trust its histogram; after
    # that, iid scores at these sizes are decided by the histogram path
    assert all(p == g.qsa.QSA_PATH_HIST for p in paths[1:]), paths
