"""q8_0 K/V (the 8-bit cache type of the runtime-tuning post, section "KV
cacheをQ8_0にしてみる") on the GPU against the CPU oracle.

- qsa_q8_0_quantize: codes and scales bit-exact (the decisions are binary32
  on both sides): random blocks over seven decades, zero blocks, .5 ties
  (power-of-two scales), binary16 subnormals and values near the binary16
  maximum, a ragged block count, and a write into the middle of a buffer
  that must leave its neighbours alone;
- qsa_gather_attend_q8_0: the oracle's attention over its own q8_0 codes
  (the same codes, checked bit for bit first) at every attention shape,
  with tails, tail-only and keep-every-block calls, and at the 256k decode
  size (255,182 tokens, 512 chosen blocks) on the rows it reads."""
import numpy as np
import pytest

import oracle
import qsagen
from parity import check_attention
from gpu_layer import GpuLayer, with_size
from qsagen import workloads as W

pytestmark = pytest.mark.gpu


def _qsa():
    import sparse_attention_decode_cache_amd as qsa
    return qsa


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _gpu_quantize(x16):
    """x16: host float16 array, last axis a multiple of 32."""
    import torch
    qsa = _qsa()
    x = _dev(x16.view(np.int16))
    codes = torch.full(x16.shape, 99, dtype=torch.int8, device="cuda")
    scales = torch.full(x16.shape[:-1] + (x16.shape[-1] // 32,), 7, dtype=torch.int16, device="cuda")
    qsa.qsa_q8_0_quantize(x, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


def _blocks(seed, n_blocks):
    rng = np.random.default_rng(seed)
    scale = 10.0 ** rng.uniform(-4, 3, size=(n_blocks, 1))
    x = rng.standard_normal((n_blocks, 32)) * scale
    x[::97] = 0.0                                           # zero blocks
    e = rng.integers(-10, 8, size=(n_blocks // 5, 1)).astype(np.float64)
    u = rng.integers(-127 * 8, 127 * 8 + 1, size=(n_blocks // 5, 32)) / 8.0
    u[:, 3] = 127.0
    x[1::5][: n_blocks // 5] = u * 2.0 ** e                 # exact .5 quotients (ties)
    x[2::11] *= 1e-4                                        # binary16 subnormals
    x[4::13] = np.clip(x[4::13] / np.abs(x[4::13]).max(axis=1, keepdims=True).clip(1e-30) * 65000,
                       -65000, 65000)                       # near the binary16 maximum
    return x.astype(np.float16)


@pytest.mark.parametrize("n_blocks", [1, 255, 257, 4099])
def test_quantize_bit_exact(n_blocks):
    x = _blocks(n_blocks, n_blocks)
    print(f"q8_0 quantize {n_blocks} blocks", flush=True)
    codes, scales = _gpu_quantize(x)
    want_c, want_s = oracle.q8_0_quantize(x)
    assert np.array_equal(scales, want_s), "scales differ"
    bad = np.argwhere(codes != want_c)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}"


def test_quantize_writes_only_its_range():
    """Rows [t0, t1) of a cache plane: the neighbours keep their bytes."""
    import torch
    qsa = _qsa()
    Hkv, Dh, cap, t0, t1 = 2, 64, 40, 13, 29
    rows = qsagen.host_normal((t1 - t0, Hkv, Dh), 4, 11, dtype=np.float16)
    codes = torch.full((cap, Hkv, Dh), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((cap, Hkv, Dh // 32), 7, dtype=torch.int16, device="cuda")
    x = _dev(rows.view(np.int16))
    qsa.qsa_q8_0_quantize(x, codes[t0:], scales[t0:], n_values=(t1 - t0) * Hkv * Dh)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    wc, ws = oracle.q8_0_quantize(rows)
    assert np.array_equal(c[t0:t1], wc) and np.array_equal(s[t0:t1], ws)
    assert np.all(c[:t0] == 99) and np.all(c[t1:] == 99)
    assert np.all(s[:t0] == 7) and np.all(s[t1:] == 7)


ATTN_SHAPES = [(4, 1, 64), (16, 2, 256), (8, 8, 64), (2, 2, 128), (8, 1, 128), (4, 4, 256)]


@pytest.mark.parametrize("Hq,Hkv,Dh", ATTN_SHAPES)
@pytest.mark.parametrize("n,k_blocks", [(1, 4), (3, 4), (4, 4), (70, 512), (2051, 512),
                                        (4097, 64), (20000, 512), (9001, 3)])
def test_gather_attend_q8_matches_oracle(Hq, Hkv, Dh, n, k_blocks):
    import torch
    qsa = _qsa()
    print(f"gather_attend_q8_0 Hq={Hq} Hkv={Hkv} Dh={Dh} n={n} K={k_blocks}", flush=True)
    rng = np.random.default_rng(n * 5 + Dh)
    K = qsagen.host_normal((n, Hkv, Dh), 10, 1 + n, dtype=np.float16)
    V = qsagen.host_normal((n, Hkv, Dh), 10, 2 + n, dtype=np.float16)
    q = qsagen.host_normal((Hq, Dh), 10, 3 + n)
    nb = n // 4
    kb = min(k_blocks, nb)
    sel = np.sort(rng.choice(nb, kb, replace=False)).astype(np.int32) if kb else np.zeros(0, np.int32)
    desc = qsa.make_desc(1, 64, qsa.QSA_F32, Hq, Hkv, Dh, 4 * k_blocks)
    cap = (n + 3) // 4 * 4
    planes = {}
    for name, X in (("k", K), ("v", V)):
        c = torch.zeros((cap, Hkv, Dh), dtype=torch.int8, device="cuda")
        s = torch.full((cap, Hkv, Dh // 32), 0x7E00, dtype=torch.int16, device="cuda")  # NaN past n
        qsa.qsa_q8_0_quantize(_dev(X.view(np.int16)), c, s)
        planes[name] = (c, s)
    kv = qsa.kv_q8_0(planes["k"][0], planes["k"][1], planes["v"][0], planes["v"][1])
    ws = qsa.workspace(desc, cap)
    out = torch.full((Hq, Dh), float("nan"), dtype=torch.float32, device="cuda")
    seld = _dev(sel) if kb else torch.zeros(1, dtype=torch.int32, device="cuda")
    qsa.qsa_gather_attend_q8_0(desc, kv, n, seld, kb, _dev(q), out, ws)
    torch.cuda.synchronize()
    Kc, Kd = oracle.q8_0_quantize(K)
    Vc, Vd = oracle.q8_0_quantize(V)
    assert np.array_equal(planes["k"][0][:n].cpu().numpy(), Kc)
    assert np.array_equal(planes["v"][1][:n].cpu().numpy().view(np.uint16), Vd)
    ref = oracle.attend_q8_0(q, Kc, Kd, Vc, Vd, oracle.cells(sel, n))
    check_attention(out.cpu().numpy(), ref)
    if kb == nb:                    # every block kept: sel may be omitted
        out2 = torch.empty_like(out)
        qsa.qsa_gather_attend_q8_0(desc, kv, n, None, nb, _dev(q), out2, ws)
        check_attention(out2.cpu().numpy(), ref)


def test_gather_attend_q8_256k():
    """The 256k decode size: 255,182 tokens (63,795 blocks, tail 2), 16 / 2
    heads x 256, 512 chosen blocks; the whole cache quantised on the GPU, the
    2,050 rows read checked against the oracle's codes and attention."""
    import torch
    qsa = _qsa()
    w = with_size(W.CTX256K, n0=255182, steps=0)
    print(f"gather_attend_q8_0 {w.name}: n={w.n0}", flush=True)
    g = GpuLayer(w)
    n, Hkv, Dh, Hq = w.n0, w.kv_heads, w.head_dim, w.q_heads
    nb = n // 4
    planes = {}
    for name, X in (("k", g.buf.k), ("v", g.buf.v)):
        c = torch.empty((g.cap, Hkv, Dh), dtype=torch.int8, device="cuda")
        s = torch.empty((g.cap, Hkv, Dh // 32), dtype=torch.int16, device="cuda")
        qsa.qsa_q8_0_quantize(X, c, s, n_values=n * Hkv * Dh)
        planes[name] = (c, s)
    kv = qsa.kv_q8_0(planes["k"][0], planes["k"][1], planes["v"][0], planes["v"][1])
    rng = np.random.default_rng(256)
    sel = np.sort(rng.choice(nb, w.k_blocks, replace=False)).astype(np.int32)
    q = qsagen.host_normal((Hq, Dh), 11, 5)
    out = torch.full((Hq, Dh), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_gather_attend_q8_0(g.desc, kv, n, _dev(sel), w.k_blocks, _dev(q), out, g.ws)
    f16 = torch.empty_like(out)
    qsa.qsa_gather_attend(g.desc, g.buf.cache, n, _dev(sel), w.k_blocks, _dev(q), f16, g.ws)
    torch.cuda.synchronize()
    cells = oracle.cells(sel, n)
    assert len(cells) == 4 * w.k_blocks + n % 4
    Kh, Vh = W.host_kv_rows(w, cells, 0)
    Kc, Kd = oracle.q8_0_quantize(Kh)
    Vc, Vd = oracle.q8_0_quantize(Vh)
    idx = torch.from_numpy(cells.astype(np.int64)).cuda()
    assert np.array_equal(planes["k"][0][idx].cpu().numpy(), Kc)
    assert np.array_equal(planes["k"][1][idx].cpu().numpy().view(np.uint16), Kd)
    assert np.array_equal(planes["v"][0][idx].cpu().numpy(), Vc)
    assert np.array_equal(planes["v"][1][idx].cpu().numpy().view(np.uint16), Vd)
    ref = oracle.attend_q8_0(q, Kc, Kd, Vc, Vd, np.arange(len(cells), dtype=np.int32))
    err = check_attention(out.cpu().numpy(), ref)
    drift = float(np.abs(out.cpu().numpy() - f16.cpu().numpy()).max())
    print(f"  max |err| {err:.2e}; q8_0 vs f16 cache max |diff| {drift:.2e}")
