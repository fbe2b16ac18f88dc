"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each group names what it pins.  Sources: post 10 by "ariera" on qiita.com
("... 長コンテキストのTGを高速化した話"), sections "QSA indexer",
"incremental pooled-key cache（COMMON-004）", "selected QSA K/V gather
（COMMON-005）", "block-domain top-k（COMMON-006）実装は見送り" and
"なぜFlash Attentionがcontext長に比例していたのか".
"""
import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ storage rounding
def test_half_conversions_match_numpy():
    """binary16 decode / RNE encode agree with numpy's IEEE conversions."""
    rng = np.random.default_rng(1)
    bits = np.arange(0, 65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    for b, v in zip(bits[::7], vals[::7]):
        got = oracle.half_to_double(b)
        assert (np.isnan(v) and np.isnan(got)) or got == v
    xs = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 1e-5, 2000), rng.normal(0, 3e4, 1000),
        # exact ties between two halves, including subnormal and overflow ties
        (vals[1000:1100] + vals[1001:1101]) / 2, np.array([65520.0, 65519.9, -65520.0, 2.0**-25, 3 * 2.0**-25]),
    ])
    for x in xs:
        want = np.float64(x).astype(np.float16).view(np.uint16)
        assert oracle.double_to_half(x) == int(want), x


# --------------------------------------------------- worked example (O1..O5)
def test_worked_example_pool_norm_rope_score():
    g = _gold("worked_example.json")
    raw = np.array(g["raw_block"] * 2, np.float32).reshape(8, 1, 4)   # blocks 0 and 1 identical
    k0 = oracle.summary_row(raw, 0, g["gamma"], g["eps"], g["theta"])[0]
    k1 = oracle.summary_row(raw, 1, g["gamma"], g["eps"], g["theta"])[0]
    np.testing.assert_allclose(k0, g["khat_block0"], rtol=2e-9)
    np.testing.assert_allclose(k1, g["khat_block1"], rtol=2e-9)
    s16 = oracle.full_summaries(raw.astype(np.float16), 2, g["gamma"], g["eps"], g["theta"])
    assert [hex(v) for v in s16[0, 0].view(np.uint16)] == g["khat_block0_f16_bits"]
    s32 = oracle.full_summaries(raw, 2, g["gamma"], g["eps"], g["theta"])
    s = oracle.scores(s32, 2, [1, 0, 0, 0], [1.0])
    np.testing.assert_allclose(s, g["score_q_e0_w1"], rtol=1e-7)
    s = oracle.scores(s32, 2, g["q2"], [g["w2"]])
    np.testing.assert_allclose(s, g["score_q2_w2"], rtol=1e-7)
    pn = [k1[0] ** 2 + k1[2] ** 2, k1[1] ** 2 + k1[3] ** 2]
    np.testing.assert_allclose(pn, g["pair_norms"], rtol=1e-8)


# ------------------------------------------------------------- pool + RMSNorm
def test_block0_is_normalised_mean_and_ms_identity():
    """At p = 0 RoPE is the identity: khat = mean / sqrt(ms + eps) * gamma, and
    (1/D) sum (khat_i / gamma_i)^2 = ms / (ms + eps)."""
    rng = np.random.default_rng(2)
    H, D, eps = 3, 8, 1e-3
    raw = rng.normal(0, 1, (4, H, D)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, D).astype(np.float32)
    k = oracle.summary_row(raw, 0, gamma, eps, 1e4)
    mean = raw.astype(np.float64).sum(0) / 4
    for h in range(H):
        ms = float(np.mean(mean[h] ** 2))
        assert np.mean((k[h] / gamma.astype(np.float64)) ** 2) == pytest.approx(ms / (ms + eps), rel=1e-13)
        np.testing.assert_allclose(k[h], mean[h] / math.sqrt(ms + eps) * gamma, rtol=1e-13)


def test_pool_uses_only_its_own_four_rows():
    rng = np.random.default_rng(3)
    raw = rng.normal(0, 1, (16, 1, 8)).astype(np.float32)
    k = oracle.summary_row(raw, 2, np.ones(8, np.float32), 1e-6, 1e4)
    raw2 = raw.copy()
    raw2[:8] = 99.0
    raw2[12:] = -7.0
    np.testing.assert_array_equal(k, oracle.summary_row(raw2, 2, np.ones(8, np.float32), 1e-6, 1e4))
    # permuting the 4 rows of the block leaves the mean unchanged
    raw3 = raw.copy()
    raw3[8:12] = raw[[11, 9, 8, 10]]
    np.testing.assert_allclose(k, oracle.summary_row(raw3, 2, np.ones(8, np.float32), 1e-6, 1e4), rtol=1e-14)


def test_rmsnorm_scale_invariance_and_gamma_per_element():
    rng = np.random.default_rng(4)
    raw = rng.normal(0, 1, (8, 2, 16)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, 16).astype(np.float32)
    a = oracle.summary_row(raw, 1, gamma, 0.0, 1e4)
    b = oracle.summary_row(raw * np.float32(8.0), 1, gamma, 0.0, 1e4)     # exact scaling
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    # gamma multiplies element i before the rotation: at p = 0 only element i moves
    g2 = gamma.copy()
    g2[5] *= 2
    a0 = oracle.summary_row(raw, 0, gamma, 1e-6, 1e4)
    b0 = oracle.summary_row(raw, 0, g2, 1e-6, 1e4)
    np.testing.assert_allclose(b0[:, 5], 2 * a0[:, 5], rtol=1e-14)
    mask = np.ones(16, bool)
    mask[5] = False
    np.testing.assert_array_equal(a0[:, mask], b0[:, mask])


# ----------------------------------------------------------------------- RoPE
@pytest.mark.parametrize("D", [2, 4, 8, 64, 128])
def test_rope_is_complex_rotation_of_half_split_pairs(D):
    """RoPE reduces to z_j * exp(i * p * theta^(-2j/D)) with z_j = x_j + i x_{j+D/2}."""
    rng = np.random.default_rng(D)
    x = rng.normal(0, 1, D)
    for pos in (0.0, 4.0, 1000.0, 255180.0):
        got = oracle.rope(x, pos, 1e4)
        half = D // 2
        for j in range(half):
            z = complex(x[j], x[j + half]) * cmath.exp(1j * pos * 1e4 ** (-2.0 * j / D))
            assert got[j] == pytest.approx(z.real, abs=1e-12)
            assert got[j + half] == pytest.approx(z.imag, abs=1e-12)
        if pos == 0.0:
            np.testing.assert_array_equal(got, x)


def test_rope_pair_norms_and_composition():
    rng = np.random.default_rng(5)
    D = 16
    x = rng.normal(0, 1, D)
    half = D // 2
    for a, b in ((4.0, 8.0), (1234.0, 255000.0)):
        ra = oracle.rope(x, a, 1e4)
        np.testing.assert_allclose(ra[:half] ** 2 + ra[half:] ** 2, x[:half] ** 2 + x[half:] ** 2, rtol=1e-12)
        np.testing.assert_allclose(oracle.rope(ra, b, 1e4), oracle.rope(x, a + b, 1e4), atol=1e-9)


def test_summary_position_is_block_start():
    """Block b is rotated at position 4b: rotating block 0's summary by 4b gives block b's."""
    rng = np.random.default_rng(6)
    blk = rng.normal(0, 1, (4, 1, 8)).astype(np.float32)
    raw = np.concatenate([blk] * 6)
    g = np.ones(8, np.float32)
    k0 = oracle.summary_row(raw, 0, g, 1e-6, 1e4)[0]
    for b in range(1, 6):
        np.testing.assert_allclose(oracle.summary_row(raw, b, g, 1e-6, 1e4)[0],
                                   oracle.rope(k0, 4.0 * b, 1e4), atol=1e-13)


# --------------------------------------------------------------------- scores
def test_scores_one_hot_weight_is_numpy_dot_and_linear():
    rng = np.random.default_rng(7)
    H, D, nb = 4, 16, 9
    summ = rng.normal(0, 1, (nb, H, D)).astype(np.float32)
    q = rng.normal(0, 1, (H, D)).astype(np.float32)
    for h in range(H):
        w = np.zeros(H, np.float32)
        w[h] = 1
        s = oracle.scores(summ, nb, q, w)
        want = [np.dot(q[h].astype(np.float64), summ[b, h].astype(np.float64)) for b in range(nb)]
        np.testing.assert_allclose(s, want, rtol=1e-13)
    w = rng.uniform(0, 1, H).astype(np.float32)
    q2 = rng.normal(0, 1, (H, D)).astype(np.float32)
    s1, s2 = oracle.scores(summ, nb, q, w), oracle.scores(summ, nb, q2, w)
    s12 = oracle.scores(summ, nb, (q.astype(np.float64) + q2).astype(np.float32), w)
    np.testing.assert_allclose(s12, s1 + s2, atol=1e-5)   # q+q2 rounded to fp32 once
    s, a = oracle.scores(summ, nb, q, w, with_scale=True)
    bound = [sum(w[h] * np.linalg.norm(q[h].astype(np.float64)) * np.linalg.norm(summ[b, h].astype(np.float64))
                 for h in range(H)) for b in range(nb)]
    assert np.all(np.abs(s) <= np.array(bound) * (1 + 1e-12))
    assert np.all(np.abs(s) <= a * (1 + 1e-12))


def test_scores_read_f16_summaries_as_stored():
    rng = np.random.default_rng(8)
    summ = rng.normal(0, 1, (5, 1, 8)).astype(np.float16)
    q = rng.normal(0, 1, 8).astype(np.float32)
    s = oracle.scores(summ, 5, q, [1.0])
    np.testing.assert_allclose(s, summ[:, 0].astype(np.float64) @ q.astype(np.float64), rtol=1e-13)


# ---------------------------------------------------------------------- top-k
def test_topk_tie_example():
    g = _gold("topk_ties.json")
    s = np.array([float(v) for v in g["scores"]])
    assert math.copysign(1, s[6]) < 0
    for k, want in g["expected"].items():
        assert oracle.topk(s, int(k)).tolist() == want


def _brute_topk(s, k):
    n = len(s)
    k = min(k, n)
    ok = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        if all((s[i] > s[j]) or (s[i] == s[j] and i < j) for i in S for j in range(n) if j not in Sset):
            ok.append(list(S))
    assert len(ok) == 1
    return ok[0]


def test_topk_exhaustive_tiny():
    rng = np.random.default_rng(9)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        s = rng.integers(-2, 3, n).astype(np.float64)   # many ties
        if trial % 3 == 0:
            s = rng.normal(0, 1, n)
        for k in range(1, n + 2):
            assert oracle.topk(s, k).tolist() == _brute_topk(list(s), k)


def test_topk_matches_lexsort():
    rng = np.random.default_rng(10)
    for n, k in ((1000, 64), (5000, 512), (300, 512), (4096, 4096)):
        s = np.round(rng.normal(0, 3, n), 1)    # ties
        want = np.sort(np.lexsort((np.arange(n), -s))[:min(k, n)])
        assert np.array_equal(oracle.topk(s, k), want)


# ---------------------------------------------------------------------- cells
def test_cells_formula_and_ceiling():
    sel = np.arange(64, dtype=np.int32) * 3
    c = oracle.cells(sel, 4097)
    assert len(c) == 257 == oracle.n_cells(4097, 64)
    assert c[-1] == 4096 and list(c[:4]) == [0, 1, 2, 3] and list(c[4:8]) == [12, 13, 14, 15]
    for n in range(1, 40):
        for k in (1, 2, 5, 512):
            kb = min(k, n // 4)
            c = oracle.cells(np.arange(kb, dtype=np.int32), n)
            assert len(c) == 4 * kb + n % 4 == oracle.n_cells(n, k)
            assert len(set(c.tolist())) == len(c) and max(c) < n
    # 2048 tokens = 512 blocks: never more than 2048 + 4 - 1 cells
    assert max(oracle.n_cells(n, 512) for n in range(2040, 2100)) == 2051
    assert oracle.n_cells(255182, 512) == 2050


# ------------------------------------------------------------------ attention
def _rand_kv(rng, T, Hkv, Dh):
    return (rng.normal(0, 1, (T, Hkv, Dh)).astype(np.float16), rng.normal(0, 1, (T, Hkv, Dh)).astype(np.float16))


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    Hq, Hkv, Dh, T = 4, 2, 16, 20
    K, V = _rand_kv(rng, T, Hkv, Dh)
    q = rng.normal(0, 1, (Hq, Dh)).astype(np.float32)
    out = oracle.attend(q, K, V, [7])
    for h in range(Hq):
        np.testing.assert_array_equal(out[h], V[7, h * Hkv // Hq].astype(np.float64))
    V2 = V.copy()
    V2[:] = V[3]
    out = oracle.attend(q, K, V2, [1, 5, 9, 11])
    for h in range(Hq):
        np.testing.assert_allclose(out[h], V[3, h * Hkv // Hq].astype(np.float64), rtol=1e-14)
    out = oracle.attend(np.zeros((Hq, Dh), np.float32), K, V, [0, 2, 4])
    for h in range(Hq):
        g = h * Hkv // Hq
        np.testing.assert_allclose(out[h], V[[0, 2, 4], g].astype(np.float64).mean(0), rtol=1e-13)


def test_sparse_equals_dense_sdpa_when_every_block_is_kept():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    Hq, Hkv, Dh = 8, 2, 32
    for n in (1, 3, 4, 37, 64):
        K, V = _rand_kv(rng, n + 5, Hkv, Dh)
        q = rng.normal(0, 1, (Hq, Dh)).astype(np.float32)
        nb = n // 4
        sel = oracle.topk(rng.normal(0, 1, nb), 512) if nb else np.zeros(0, np.int32)
        c = oracle.cells(sel, n)
        assert sorted(c.tolist()) == list(range(n))
        out = oracle.attend(q, K, V, c)
        Kt = torch.from_numpy(K[:n].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        Vt = torch.from_numpy(V[:n].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        qt = torch.from_numpy(q.astype(np.float64)).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous())
        np.testing.assert_allclose(out, ref.squeeze(1).numpy(), rtol=1e-12, atol=1e-13)


def test_attention_cell_order_does_not_matter():
    rng = np.random.default_rng(13)
    K, V = _rand_kv(rng, 50, 1, 16)
    q = rng.normal(0, 1, (2, 16)).astype(np.float32)
    c = np.array([3, 8, 9, 40, 41, 2], np.int32)
    np.testing.assert_allclose(oracle.attend(q, K, V, c), oracle.attend(q, K, V, c[::-1].copy()), rtol=1e-13)


# ------------------------------------------------------------------ watermark
def _layer(rng, cap, n0, H=2, D=8, dtype=np.float16, k_blocks=3):
    raw = rng.normal(0, 1, (cap, H, D)).astype(dtype)
    K, V = _rand_kv(rng, cap, 1, 8)
    gamma = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return oracle.OracleLayer(raw, K, V, gamma, 1e-6, 1e4, n0, k_blocks)


def test_incremental_equals_full_rebuild_after_every_append():
    rng = np.random.default_rng(14)
    for dtype in (np.float16, np.float32):
        L = _layer(rng, 64, 5, dtype=dtype)
        L.rebuild()
        for t in range(5, 60):
            r = L.step(rng.normal(0, 1, (2, 8)).astype(dtype), rng.normal(0, 1, (1, 8)).astype(np.float16),
                       rng.normal(0, 1, (1, 8)).astype(np.float16), rng.normal(0, 1, 16).astype(np.float32),
                       rng.uniform(0, 1, 2).astype(np.float32), rng.normal(0, 1, (2, 8)).astype(np.float32))
            nb = L.n // 4
            full = oracle.full_summaries(L.raw[:L.n], nb, L.gamma, L.eps, L.theta)
            assert np.array_equal(L.summary[:nb].view(np.uint8), full.view(np.uint8))
            assert len(r["cells"]) == oracle.n_cells(L.n, 3)


def test_invalidate_and_truncate_rebuild():
    rng = np.random.default_rng(15)
    L = _layer(rng, 128, 100)
    L.rebuild()
    ref = L.summary.copy()
    for pos in (0, 3, 50, 97, 99, 400):
        L.summary[pos // 4:] = 0            # distrusted rows may hold anything
        L.invalidate(pos)
        assert L.valid == min(25, pos // 4)
        L.rebuild()
        assert np.array_equal(L.summary.view(np.uint16), ref.view(np.uint16))
    # sequence edit at 61: tokens >= 61 are dropped and different ones appended
    L.truncate(61)
    assert L.n == 61 and L.valid == 15
    for t in range(61, 90):
        L.append(rng.normal(0, 1, (2, 8)).astype(np.float16), L.K[0], L.V[0])
    L.rebuild()
    fresh = oracle.full_summaries(L.raw[:90], 22, L.gamma, L.eps, L.theta)
    assert np.array_equal(L.summary[:22].view(np.uint16), fresh.view(np.uint16))
    assert not np.array_equal(L.summary[15:22].view(np.uint16), ref[15:22].view(np.uint16))
