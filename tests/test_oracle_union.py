"""Pins of the oracle's grouped-union attention (a reading of post 10's
"QSA grouped-union": a group of consecutive queries reads the union of its
cells once and each query attends over it with the cells that are not its
own masked out).  Pinned against what fixes it independently: set union by
Python sets, the per-query attention of the oracle (itself pinned against
torch's SDPA), and a pure-Python masked softmax on a tiny case."""
import math

import numpy as np

import oracle


def _rand_sels(rng, nq, nb_of, k):
    sels = []
    for i in range(nq):
        nb = nb_of(i)
        kk = min(k, nb)
        sels.append(np.sort(rng.choice(nb, size=kk, replace=False)).astype(np.int32))
    return sels


def test_union_blocks_is_the_set_union():
    rng = np.random.default_rng(11)
    for trial in range(20):
        nq = int(rng.integers(1, 9))
        sels = _rand_sels(rng, nq, lambda i: 40 + i, int(rng.integers(1, 30)))
        want = sorted(set().union(*[set(x.tolist()) for x in sels]))
        assert oracle.union_blocks(sels).tolist() == want
    same = np.arange(5, 25, 2, dtype=np.int32)
    assert np.array_equal(oracle.union_blocks([same, same, same]), same)          # identical: the list
    a, b = np.array([1, 4, 9], np.int32), np.array([2, 3, 10, 11], np.int32)
    assert np.array_equal(oracle.union_blocks([a, b]), np.sort(np.concatenate([a, b])))   # disjoint


def test_union_attend_is_each_querys_own_attention():
    rng = np.random.default_rng(12)
    Hq, Hkv, Dh = 4, 2, 16
    n0 = 61
    nq = 6
    ntok = n0 + nq
    K = rng.standard_normal((ntok, Hkv, Dh)).astype(np.float16)
    V = rng.standard_normal((ntok, Hkv, Dh)).astype(np.float16)
    q = rng.standard_normal((nq, Hq, Dh)).astype(np.float32)
    n = [n0 + i + 1 for i in range(nq)]
    sels = _rand_sels(rng, nq, lambda i: n[i] // 4, 5)
    got = oracle.union_attend(q, K, V, sels, n)
    for i in range(nq):
        ref = oracle.attend(q[i], K, V, oracle.cells(sels[i], n[i]))
        assert np.max(np.abs(got[i] - ref)) < 1e-12


def test_union_attend_tiny_by_hand():
    # two queries, 1 head, Dh 2: blocks of 4 cells, tails, masks written out
    rng = np.random.default_rng(13)
    ntok = 14
    K = rng.standard_normal((ntok, 1, 2)).astype(np.float16)
    V = rng.standard_normal((ntok, 1, 2)).astype(np.float16)
    q = rng.standard_normal((2, 1, 2)).astype(np.float32)
    n = [10, 13]                          # query 0: blocks 0, 1 complete, tail 8, 9; query 1: + block 2, tail 12
    sels = [np.array([1], np.int32), np.array([0, 2], np.int32)]
    got = oracle.union_attend(q, K, V, sels, n)
    own = [list(range(4, 8)) + [8, 9], list(range(0, 4)) + list(range(8, 12)) + [12]]
    for i in range(2):
        lg = [float(q[i, 0, 0]) * float(K[c, 0, 0]) / math.sqrt(2) + float(q[i, 0, 1]) * float(K[c, 0, 1]) / math.sqrt(2)
              for c in own[i]]
        mx = max(lg)
        wts = [math.exp(x - mx) for x in lg]
        z = sum(wts)
        for d in range(2):
            ref = sum(w * float(V[c, 0, d]) for w, c in zip(wts, own[i])) / z
            assert abs(got[i, 0, d] - ref) < 1e-12
