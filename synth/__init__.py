"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no arithmetic of the method: it only draws routing splits and
bf16 tensors. NumPy PCG64, one generator per tensor; normals are drawn in
fp32 and rounded to bf16 (round to nearest even) on the host, so the device
path and the oracle see identical bits.

Workloads (MoE expert layers; every split vector sums to the row count):

* ``tiny``      4 experts, splits [64, 0, 96, 96], K = N = 256.
* ``fc1``       32 experts, 4096 tokens x top-8 = 32768 rows, splits from a
                Dirichlet(0.5) probability vector with 3 experts forced to
                zero, multinomial counts; K = 4096, N = 3072 (gated FFN FC1).
* ``a8w4``      128 experts, 8192 tokens x top-8 = 65536 rows, heavy-tailed
                (Zipf s = 1.1 over a random expert order) with 8 experts
                forced to zero; K = 7168, N = 2048.
* ``blockwise`` 64 experts, 32768 rows, uniform-random routing read as
                Dirichlet(1) probabilities and multinomial counts;
                K = 7168, N = 4096.
"""
from __future__ import annotations

import numpy as np

SEED_SPLITS, SEED_A, SEED_W, SEED_DY, SEED_MAIN_GRAD = 0, 1, 2, 3, 4

__all__ = [
    "SEED_SPLITS", "SEED_A", "SEED_W", "SEED_DY", "SEED_MAIN_GRAD",
    "WORKLOADS", "fp32_to_bf16_bits", "bf16_normal", "f32_normal",
    "splits_dirichlet", "splits_zipf", "splits_for",
]


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_normal(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) samples (fp32 draw, RNE to bf16)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return fp32_to_bf16_bits(x)


def f32_normal(shape, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float32)


def splits_dirichlet(G: int, M: int, alpha: float, n_zero: int, seed: int) -> np.ndarray:
    """Counts ~ Multinomial(M, p), p ~ Dirichlet(alpha), n_zero experts forced to 0."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(G, alpha))
    if n_zero:
        p[rng.choice(G, size=n_zero, replace=False)] = 0.0
    p = p / p.sum()
    return rng.multinomial(M, p).astype(np.int64)


def splits_zipf(G: int, M: int, s: float, n_zero: int, seed: int) -> np.ndarray:
    """Counts ~ Multinomial(M, p) with p_rank ∝ rank^-s over a random expert
    order and n_zero experts forced to 0."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(G)
    p = np.empty(G)
    p[order] = 1.0 / np.arange(1, G + 1, dtype=np.float64) ** s
    if n_zero:
        p[rng.choice(G, size=n_zero, replace=False)] = 0.0
    p = p / p.sum()
    return rng.multinomial(M, p).astype(np.int64)


WORKLOADS = {
    "tiny": dict(G=4, M=256, K=256, N=256, w_std=1.0),
    "fc1": dict(G=32, M=32768, K=4096, N=3072, w_std=0.02),
    "a8w4": dict(G=128, M=65536, K=7168, N=2048, w_std=0.02),
    "blockwise": dict(G=64, M=32768, K=7168, N=4096, w_std=0.02),
}


def splits_for(name: str, seed: int = SEED_SPLITS) -> np.ndarray:
    w = WORKLOADS[name]
    if name == "tiny":
        return np.array([64, 0, 96, 96], dtype=np.int64)
    if name == "fc1":
        return splits_dirichlet(w["G"], w["M"], 0.5, 3, seed)
    if name == "a8w4":
        return splits_zipf(w["G"], w["M"], 1.1, 8, seed)
    if name == "blockwise":
        return splits_dirichlet(w["G"], w["M"], 1.0, 0, seed)
    raise KeyError(name)
