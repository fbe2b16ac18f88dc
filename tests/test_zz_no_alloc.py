"""qsa_decode_step_static (no workspace argument, a static device array as
its workspace) against qsa_decode_step with a workspace: the same inputs
give the same ids and scores bit for bit and outputs within the attention
tolerance, on two calls in a row (steps of a 64k-token layer, then of a
smaller 20k-token layer, so that the second call finds the first one's
contents in the static array)."""
import numpy as np
import pytest

from gpu_layer import GpuLayer, with_size
from parity import ATTN_ATOL
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _static_step(g, s):
    q = g.qsa
    q.qsa_decode_step_static(g.desc, g.buf.cache, g.state, g.inp.raw[s], g.inp.k[s], g.inp.v[s], g.gamma,
                             g.inp.q_idx[s], g.inp.w[s], g.inp.q[s], g.out, g.sel, g.scores)
    nb = g.state.n_tokens // 4
    return {"n": g.state.n_tokens, "out": g.out.cpu().numpy().astype(np.float64),
            "sel": g.sel[:min(g.w.k_blocks, nb)].cpu().numpy(), "scores": g.scores[:nb].cpu().numpy()}


def test_static_workspace_matches_workspace_entry():
    for w in (with_size(W.CTX64K, steps=3), with_size(W.CTX64K, n0=20011, steps=3)):
        print(f"static decode {w.name} n0={w.n0}", flush=True)
        a = GpuLayer(w)
        b = GpuLayer(w)
        for s in range(w.steps):
            ra = a.step(s)
            rb = _static_step(b, s)
            assert ra["n"] == rb["n"]
            assert np.array_equal(ra["sel"], rb["sel"])
            assert np.array_equal(ra["scores"].view(np.uint32), rb["scores"].view(np.uint32))
            err = float(np.max(np.abs(ra["out"] - rb["out"])))
            assert err <= ATTN_ATOL, err
