"""The seeded input generator (host side).  It is shared by both paths and
holds none of the attention method's arithmetic."""
import numpy as np

import qsagen


def test_splitmix64_known_answers():
    # published splitmix64 sequence for seed 1234567 (state advances by the golden gamma)
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    x = 1234567
    for w in want:
        assert qsagen.mix(x) == w
        x = (x + 0x9E3779B97F4A7C15) % 2**64


def test_normal_is_exact_fixed_point_and_deterministic():
    a = qsagen.host_normal((4096, 8), 7, qsagen.tensor_id(qsagen.KIND_RAW))
    b = qsagen.host_normal((4096, 8), 7, qsagen.tensor_id(qsagen.KIND_RAW))
    assert np.array_equal(a, b)
    assert np.all(np.abs(a) <= 6.0)
    assert np.array_equal(a * 65536, np.round(a * 65536))          # multiples of 2^-16
    assert abs(a.mean()) < 0.03 and abs(a.var() - 1.0) < 0.03
    c = qsagen.host_normal((4096, 8), 7, qsagen.tensor_id(qsagen.KIND_K))
    assert not np.array_equal(a, c)
    # row access and offset access give the same bits as the full tensor
    rows = qsagen.host_rows([5, 100, 4095], (8,), 7, qsagen.tensor_id(qsagen.KIND_RAW))
    assert np.array_equal(rows, a[[5, 100, 4095]])
    off = qsagen.host_normal((10, 8), 7, qsagen.tensor_id(qsagen.KIND_RAW), e0=8 * 100)
    assert np.array_equal(off, a[100:110])
    h = qsagen.host_normal((64,), 7, 3, dtype=np.float16)
    assert np.array_equal(h, qsagen.host_normal((64,), 7, 3).astype(np.float16))


def test_unit():
    u = qsagen.host_unit((100000,), 1, 2)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    assert np.array_equal(u * 2**23, np.round(u * 2**23))
    g = qsagen.host_unit((1000,), 1, 2, offset=0.5)
    assert np.array_equal(g, np.float32(0.5) + u[:1000])
