"""Pins of the oracle's q8_0 K/V functions (CPU only).

q8_0 (llama.cpp's 8-bit cache type, tried on the runtime-tuning post,
section "KV cacheをQ8_0にしてみる"): 32 consecutive values share one binary16
scale s = amax / 127 and are stored as round(x / s) with halves away from
zero, the decisions taken in binary32.  Each pin below fixes the result by
something other than the oracle's own code: blocks whose scale is a power of
two (every step exact, so the codes are the rounded quotients themselves), a
block checked by hand, sign and power-of-two symmetry, the error bound of
rounding to the nearest code, and for the attention a reduction to the
already pinned f16 attention and to torch's attention in float64."""
import numpy as np
import pytest

import oracle


def _round_away(u):
    return np.where(u >= 0, np.floor(u + 0.5), -np.floor(-u + 0.5))


def _pow2_blocks(rng, n_blocks, exps, grid=8):
    """Blocks x = u * 2^e with u on a 1/grid grid in [-127, 127] (one |u| =
    127): amax / 127 = 2^e exactly, so codes = round_away(u), scale = 2^e
    (grid 1: integer u, so the codes decode to x exactly)."""
    u = rng.integers(-127 * grid, 127 * grid + 1, size=(n_blocks, 32)) / float(grid)
    u[np.arange(n_blocks), rng.integers(0, 32, n_blocks)] = 127.0 * rng.choice([-1, 1], n_blocks)
    e = np.asarray(exps, np.float64)[:, None]
    x = (u * 2.0 ** e).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), u * 2.0 ** e), "construction not exact in f16"
    return x, u, e[:, 0]


def test_power_of_two_scales_give_the_rounded_quotients():
    rng = np.random.default_rng(5)
    exps = rng.integers(-12, 9, size=64)
    x, u, e = _pow2_blocks(rng, 64, exps)
    codes, d = oracle.q8_0_quantize(x)
    assert np.array_equal(codes.astype(np.float64), _round_away(u))
    assert np.array_equal(d[:, 0].view(np.float16).astype(np.float64), 2.0 ** e)
    # the grid holds .5 quotients of both parities: halves go away from zero
    assert np.any(np.isclose(np.abs(u) % 2, 0.5)) and np.any(np.isclose(np.abs(u) % 2, 1.5))


def test_hand_checked_block():
    """amax 127 -> scale 1.0 (0x3c00); 2.5 -> 3, -2.5 -> -3, 62.5 -> 63,
    0.5 -> 1, 1.5 -> 2, 0.25 -> 0, -0.75 -> -1 (ties away from zero, not to even)."""
    x = np.zeros(32, np.float16)
    x[:9] = [127, 2.5, -2.5, 62.5, 0.5, -0.5, 1.5, 0.25, -0.75]
    codes, d = oracle.q8_0_quantize(x)
    assert codes[:9].tolist() == [127, 3, -3, 63, 1, -1, 2, 0, -1]
    assert np.all(codes[9:] == 0) and d.tolist() == [0x3C00]


def test_zero_block_and_block_independence():
    x = np.zeros((3, 32), np.float16)
    x[0, 5] = -4.0          # scale 4/127, the -4 maps to -127
    x[2, 31] = 0.0078125    # a small block beside it
    codes, d = oracle.q8_0_quantize(x)
    assert codes[0, 5] == -127 and np.all(np.delete(codes[0], 5) == 0)
    assert np.all(codes[1] == 0) and d[1, 0] == 0
    assert codes[2, 31] == 127 and np.all(codes[2, :31] == 0)
    assert d[0, 0] == np.float16(4.0 / 127).view(np.uint16)


def test_error_bound_symmetry_and_ceiling():
    rng = np.random.default_rng(9)
    scales = 10.0 ** rng.uniform(-3, 2, size=(200, 1))
    x = (rng.standard_normal((200, 32)) * scales).astype(np.float16)
    codes, d = oracle.q8_0_quantize(x)
    xf = x.astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    s = amax / 127.0
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=1) == 127)
    # nearest code: |x - code s| <= s/2 (up to the binary32 quotient's rounding)
    err = np.abs(xf - codes * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # the stored scale is s rounded to binary16
    assert np.array_equal(d[:, 0], s.astype(np.float32).astype(np.float16).view(np.uint16))
    # sign symmetry and power-of-two scaling
    c2, d2 = oracle.q8_0_quantize(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(d2, d)
    c3, d3 = oracle.q8_0_quantize((xf * 4).astype(np.float16))
    assert np.array_equal(c3, codes)
    normal = s >= 2.0 ** -14          # binary16 subnormal scales lose bits, so 4x is exact only above
    assert normal.sum() > 100
    assert np.array_equal(d3[normal].view(np.float16).astype(np.float64),
                          d[normal].view(np.float16).astype(np.float64) * 4)


def test_values_decode_per_32_value_block():
    codes = np.arange(-64, 64, dtype=np.int8).reshape(2, 64)
    d = np.array([[0x3C00, 0x4000], [0x3800, 0x0000]], np.uint16)   # 1, 2, 0.5, 0
    v = oracle.q8_0_values(codes, d)
    want = codes.astype(np.float64) * np.repeat([[1.0, 2.0], [0.5, 0.0]], 32, axis=1)
    assert np.array_equal(v, want)


def _q8_cache(rng, n, Hkv, Dh, exact):
    if exact:       # power-of-two scales: the codes decode to the f16 values exactly
        nblk = n * Hkv * Dh // 32
        K, _, _ = _pow2_blocks(rng, nblk, rng.integers(-9, -5, nblk), grid=1)
        V, _, _ = _pow2_blocks(rng, nblk, rng.integers(-9, -5, nblk), grid=1)
        K, V = K.reshape(n, Hkv, Dh), V.reshape(n, Hkv, Dh)
    else:
        K = rng.standard_normal((n, Hkv, Dh)).astype(np.float16)
        V = rng.standard_normal((n, Hkv, Dh)).astype(np.float16)
    Kc, Kd = oracle.q8_0_quantize(K)
    Vc, Vd = oracle.q8_0_quantize(V)
    return K, V, Kc, Kd, Vc, Vd


@pytest.mark.parametrize("Hq,Hkv,Dh", [(4, 1, 64), (16, 2, 256), (2, 2, 128)])
def test_attend_q8_equals_f16_attend_on_exact_values(Hq, Hkv, Dh):
    rng = np.random.default_rng(Dh + Hq)
    n = 23
    K, V, Kc, Kd, Vc, Vd = _q8_cache(rng, n, Hkv, Dh, exact=True)
    assert np.array_equal(oracle.q8_0_values(Kc, Kd), K.astype(np.float64))
    q = rng.standard_normal((Hq, Dh)).astype(np.float32)
    cells = np.array([0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22], np.int32)
    a = oracle.attend_q8_0(q, Kc, Kd, Vc, Vd, cells)
    b = oracle.attend(q, K, V, cells)
    assert np.array_equal(a, b)


def test_attend_q8_matches_torch_float64():
    import torch
    rng = np.random.default_rng(17)
    n, Hq, Hkv, Dh = 37, 8, 2, 64
    _, _, Kc, Kd, Vc, Vd = _q8_cache(rng, n, Hkv, Dh, exact=False)
    q = rng.standard_normal((Hq, Dh)).astype(np.float32)
    got = oracle.attend_q8_0(q, Kc, Kd, Vc, Vd, np.arange(n, dtype=np.int32))
    Kv = torch.from_numpy(oracle.q8_0_values(Kc, Kd))            # [n, Hkv, Dh]
    Vv = torch.from_numpy(oracle.q8_0_values(Vc, Vd))
    G = Hq // Hkv
    Kh = Kv.permute(1, 0, 2).repeat_interleave(G, 0)            # [Hq, n, Dh]
    Vh = Vv.permute(1, 0, 2).repeat_interleave(G, 0)
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]     # [Hq, 1, Dh]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kh, Vh)[:, 0, :].numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12
