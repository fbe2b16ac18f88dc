"""Each HIP stage alone against the CPU oracle on identical seeded inputs.

Sizes span several workgroup tiles and a ragged tail; shapes cover every
supported indexer row layout and attention shape.
"""
import numpy as np
import pytest

import oracle
import qsagen
from parity import check_attention, check_scores, check_summaries
from gpu_layer import GpuLayer, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _qsa():
    import sparse_attention_decode_cache_amd as qsa
    return qsa


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------- stage 1: pool
@pytest.mark.parametrize("w", [with_size(W.TINY, n0=4096 + 3, steps=0),
                               with_size(W.CTX64K, n0=8192 + 2, steps=0),
                               with_size(W.CTX64K, n0=1001, steps=0, idx_heads=1, idx_dim=64),
                               with_size(W.TINY, n0=2050, steps=0, idx_heads=4, idx_dim=64)],
                         ids=["tiny-f32-1x64", "f16-4x128", "f16-1x64", "f32-4x64"])
def test_cache_update_matches_oracle(w):
    print(f"cache_update {w.name} n0={w.n0} H={w.idx_heads} D={w.idx_dim} f16={w.idx_f16}", flush=True)
    g = GpuLayer(w)
    nb = w.n0 // 4
    got = g.buf.summary[:nb].cpu().numpy()
    raw = W.host_raw_rows(w, np.arange(4 * nb), 0)
    ref = oracle.full_summaries(raw, nb, W.host_gamma(w, 0), w.rms_eps, w.rope_theta)
    ndiff = check_summaries(got, ref)
    print(f"  {ndiff} of {got.size} elements differ by one ulp")
    assert ndiff <= got.size // 1000
    # a second build of a sub-range is bitwise identical (idempotent)
    qsa = _qsa()
    qsa.qsa_cache_update(g.desc, g.buf.cache, g.gamma, nb // 3, nb)
    assert np.array_equal(g.buf.summary[:nb].cpu().numpy().view(np.uint8), got.view(np.uint8))


# ------------------------------------------------------------ stage 2: score
ROW_SHAPES = [(1, 64, False), (1, 128, False), (4, 64, False),
              (1, 64, True), (1, 128, True), (4, 64, True), (4, 128, True)]


@pytest.mark.parametrize("H,D,f16", ROW_SHAPES)
@pytest.mark.parametrize("nb", [1, 63, 64, 65, 257, 4099])
def test_index_score_matches_oracle(H, D, f16, nb):
    import torch
    qsa = _qsa()
    print(f"index_score H={H} D={D} f16={f16} nb={nb}", flush=True)
    dt = np.float16 if f16 else np.float32
    summ = qsagen.host_normal((nb, H, D), 5, 100 + nb, dtype=dt)
    q = qsagen.host_normal((H, D), 5, 200 + nb)
    wt = qsagen.host_unit((H,), 5, 300 + nb)
    desc = qsa.make_desc(H, D, qsa.QSA_F16 if f16 else qsa.QSA_F32, 4, 1, 64, 256)
    cap = 4 * nb
    sd = _dev(summ)
    cache = qsa.qsa_layer_cache(0, sd.data_ptr(), 0, 0, cap)
    out = torch.full((nb + 1,), 7.0, dtype=torch.float32, device="cuda")
    qsa.qsa_index_score(desc, cache, nb, _dev(q), _dev(wt), out)
    got = out.cpu().numpy()
    assert got[nb] == 7.0          # nothing written past n_blocks
    ref, scale = oracle.scores(summ, nb, q, wt, with_scale=True)
    err = check_scores(got[:nb], ref, scale)
    assert err < 1e-5               # fp32 accumulation is far inside the tolerance


# ------------------------------------------------------------ stage 3: top-k
def _topk_cases():
    rng = np.random.default_rng(0)
    yield "normal-63795", rng.normal(0, 13, 63795).astype(np.float32), 512
    yield "normal-513", rng.normal(0, 1, 513).astype(np.float32), 512
    yield "normal-1025", rng.normal(0, 1, 1025).astype(np.float32), 512
    yield "normal-4099-k64", rng.normal(0, 1, 4099).astype(np.float32), 64
    yield "k1", rng.normal(0, 1, 3000).astype(np.float32), 1
    yield "all-equal", np.full(5000, 1.25, np.float32), 512
    yield "all-zero-signed", np.where(rng.random(5000) < 0.5, -0.0, 0.0).astype(np.float32), 512
    yield "few-levels", rng.integers(-3, 4, 20000).astype(np.float32), 512
    yield "ties-at-threshold", np.concatenate([np.full(500, 9.0), np.full(3000, 5.0), np.zeros(10000)]).astype(np.float32), 512
    yield "denormals", (rng.integers(-50, 50, 6000) * np.float32(1e-42)).astype(np.float32), 512
    yield "huge", (rng.uniform(-1, 1, 6000) * 3e38).astype(np.float32), 512
    yield "one-bin", (1.0 + rng.integers(0, 2**10, 70000) * np.float32(2.0**-23)).astype(np.float32), 512
    yield "sorted-desc", np.sort(rng.normal(0, 1, 9000)).astype(np.float32)[::-1].copy(), 512
    yield "n-eq-k", rng.normal(0, 1, 512).astype(np.float32), 512
    yield "n-lt-k", rng.normal(0, 1, 100).astype(np.float32), 512


@pytest.mark.parametrize("name,scores,k", list(_topk_cases()), ids=[c[0] for c in _topk_cases()])
def test_topk_bit_exact_on_identical_scores(name, scores, k):
    import torch
    qsa = _qsa()
    n = scores.shape[0]
    print(f"topk_blocks {name} n={n} k={k}", flush=True)
    desc = qsa.make_desc(4, 128, qsa.QSA_F16, 16, 2, 256, 2048)
    ws = qsa.workspace(desc, 4 * n)
    sel = torch.full((min(k, n) + 1,), -7, dtype=torch.int32, device="cuda")
    s_dev = _dev(scores)
    for rep in range(2):            # bitwise repeatable
        qsa.qsa_topk_blocks(s_dev, n, k, sel, ws)
        got = sel.cpu().numpy()
        want = oracle.topk(scores.astype(np.float64), k)
        assert got[-1] == -7
        assert np.array_equal(got[:-1], want), f"rep {rep}"


# ---------------------------------------------------------- stage 4: attend
ATTN_SHAPES = [(4, 1, 64), (16, 2, 256), (8, 8, 64), (2, 2, 128), (8, 1, 128), (4, 4, 256)]


@pytest.mark.parametrize("Hq,Hkv,Dh", ATTN_SHAPES)
@pytest.mark.parametrize("n,k_blocks", [(1, 4), (3, 4), (4, 4), (7, 64), (70, 512), (2051, 512),
                                        (4097, 64), (20000, 512), (9001, 3)])
def test_gather_attend_matches_oracle(Hq, Hkv, Dh, n, k_blocks):
    import torch
    qsa = _qsa()
    print(f"gather_attend Hq={Hq} Hkv={Hkv} Dh={Dh} n={n} K={k_blocks}", flush=True)
    rng = np.random.default_rng(n * 7 + Dh)
    K = qsagen.host_normal((n, Hkv, Dh), 9, 1 + n, dtype=np.float16)
    V = qsagen.host_normal((n, Hkv, Dh), 9, 2 + n, dtype=np.float16)
    q = qsagen.host_normal((Hq, Dh), 9, 3 + n)
    nb = n // 4
    kb = min(k_blocks, nb)
    sel = np.sort(rng.choice(nb, kb, replace=False)).astype(np.int32) if kb else np.zeros(0, np.int32)
    desc = qsa.make_desc(1, 64, qsa.QSA_F32, Hq, Hkv, Dh, 4 * k_blocks)
    cap = (n + 3) // 4 * 4
    Kd = torch.zeros((cap, Hkv, Dh), dtype=torch.float16, device="cuda")
    Vd = torch.zeros_like(Kd)
    Kd[:n] = _dev(K)
    Vd[:n] = _dev(V)
    if cap > n:
        Kd[n:] = float("nan")
        Vd[n:] = float("nan")
    cache = qsa.qsa_layer_cache(0, 0, Kd.data_ptr(), Vd.data_ptr(), cap)
    ws = qsa.workspace(desc, cap)
    out = torch.empty((Hq, Dh), dtype=torch.float32, device="cuda")
    seld = _dev(sel) if kb else torch.zeros(1, dtype=torch.int32, device="cuda")
    qsa.qsa_gather_attend(desc, cache, n, seld, kb, _dev(q), out, ws)
    ref = oracle.attend(q, K, V, oracle.cells(sel, n))
    check_attention(out.cpu().numpy(), ref)
    if kb == nb:                    # every block kept: sel may be omitted
        out2 = torch.empty_like(out)
        qsa.qsa_gather_attend(desc, cache, n, None, nb, _dev(q), out2, ws)
        check_attention(out2.cpu().numpy(), ref)
