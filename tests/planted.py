"""Planted inputs: blocks whose scores are graded so that the k-th and
(k+1)-th largest block scores differ by a known relative gap.

Independent random keys put the k-th / (k+1)-th gap far below the top-k
rule's 1e-3 threshold, so the rule's exact branch (ids compared bit for bit
with the oracle's) is never taken on them.  Here N_PLANT blocks get raw key
rows built backwards through the pooled-key pipeline of post 10 ("QSAとQSA
indexerについて": mean of 4 rows -> per-head RMSNorm with gamma -> RoPE at
the block's first position) so that their pooled, normalised, rotated key
has a chosen component T_i along a fixed unit direction u_h in every head;
the query of every step is q_idx_h = sqrt(D) u_h with fixed head weights w,
so block i scores sqrt(D) T_i sum_h w_h (the same order whatever w is).  The
T_i fall geometrically by GAP per rank around rank k and stay far above any
score of the random blocks.

This is test infrastructure: the construction uses the oracle's RoPE for
the inverse rotation and is checked against the oracle's own scores in
tests/test_planted.py.
"""
import dataclasses

import numpy as np

import oracle
from qsagen import workloads as W

N_PLANT = 600
GAP = 3e-3                  # relative gap between consecutive ranks around rank k
T_K = 5.5                   # component along u_h of the k-th block's key (per head)
T_TOP = 9.0                 # of the top block
SEED = 0x51534150           # numpy generator seed of the directions and the noise


@dataclasses.dataclass
class Planted:
    blocks: np.ndarray      # [N] planted block ids (ascending)
    rank: np.ndarray        # [N] rank of each (0 = highest score)
    rows: np.ndarray        # [N, 4, H, D] raw key rows of each block (storage dtype)
    q_idx: np.ndarray       # [H, D] fp32, every step
    w: np.ndarray           # [H] fp32, every step


def targets(k, n=N_PLANT):
    """T_i for ranks 0 .. n-1: geometric with ratio 1 + GAP over the 32 ranks
    above rank k - 1 and everything below it, linear above that."""
    t = np.empty(n)
    for i in range(n):
        if i >= k - 33:
            t[i] = T_K * (1.0 + GAP) ** (k - 1 - i)
    top = k - 33
    if top > 0:
        hi = T_TOP if T_TOP > t[top] else t[top] * 1.5
        t[:top] = np.linspace(hi, t[top], top + 1)[:top]
    return t


def make(w, layer, seq=0, n=N_PLANT, k=None):
    """The planted rows of layer `layer` of workload w (blocks spread evenly
    over the prefilled ones, ranks a seeded permutation)."""
    k = k or w.k_blocks
    H, D = w.idx_heads, w.idx_dim
    nb0 = w.n0 // 4
    assert nb0 >= n and n > k
    dt = np.float16 if w.idx_f16 else np.float32
    rng = np.random.default_rng(SEED + 7919 * layer + 104729 * seq)
    gamma = W.host_gamma(w, layer, seq).astype(np.float64)
    u = rng.standard_normal((H, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    blocks = ((np.arange(n) + 0.5) * nb0 / n).astype(np.int64)
    rank = rng.permutation(n)
    t = targets(k, n)[rank]
    rows = np.empty((n, 4, H, D), dt)
    for j in range(n):
        b = int(blocks[j])
        for h in range(H):
            noise = rng.standard_normal(D)
            noise -= noise.dot(u[h]) * u[h]
            noise /= np.linalg.norm(noise)
            c = min(0.99, t[j] / (np.sqrt(D) / 1.155))
            for _ in range(5):
                z = c * u[h] + np.sqrt(1.0 - c * c) * noise
                x = np.sqrt(D) * oracle.rope(z, -4.0 * b, w.rope_theta) / gamma
                xs = x.astype(dt).astype(np.float64)
                y = xs / np.sqrt(np.mean(xs * xs) + w.rms_eps) * gamma
                got = oracle.rope(y, 4.0 * b, w.rope_theta).dot(u[h])
                c = min(0.999, c * t[j] / got)
            rows[j, :, h] = xs.astype(dt)
    q_idx = (np.sqrt(D) * u).astype(np.float32)
    wt = W.host_step_inputs(w, layer, 0, seq)[1]
    return Planted(blocks, rank, rows, q_idx, wt)


def apply_host(p, raw):
    """Write the planted rows into a host raw-key array [tokens, H, D]."""
    for j, b in enumerate(p.blocks):
        raw[4 * b:4 * b + 4] = p.rows[j]


def apply_device(p, idx_k):
    """Write the planted rows into a device raw-key tensor [capacity, H, D]."""
    import torch
    idx = torch.as_tensor((4 * p.blocks[:, None] + np.arange(4)[None, :]).reshape(-1), device=idx_k.device)
    src = torch.from_numpy(p.rows.reshape((-1,) + p.rows.shape[2:])).to(idx_k.device)
    idx_k[idx] = src
