"""Mean-pooled block proxy scores, float64.

SCOPE abstract: training-free sparse attention commonly predicts its mask from
block-level proxy scores instead of the full attention map.  The proxy used
here pools each block of B consecutive tokens by its mean -- the same block
aggregation as ScalingAttention Eq. 1, applied to Q and K instead of the
attention map -- and scores a block pair with the scaled inner product of the
pooled vectors:

    qbar_u = mean_{i in block u, i < N} q_i,   kbar_v = mean_{j in block v, j < N} k_j
    S[u, v] = scale * <qbar_u, kbar_v>

The last block averages only its real tokens.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def block_means(x: np.ndarray, block: int = 64) -> np.ndarray:
    """[H, N, d] -> [H, nb, d] float64 means over the real tokens of each block."""
    H, n, d = x.shape
    nb = -(-n // block)
    out = np.empty((H, nb, d), np.float64)
    for u in range(nb):
        out[:, u] = np.asarray(x[:, u * block: min(n, (u + 1) * block)], np.float64).mean(axis=1)
    return out


def block_scores(q: np.ndarray, k: np.ndarray, scale: float, block: int = 64) -> np.ndarray:
    """[H, nb, nb] float64 scores."""
    qb = block_means(q, block)
    kb = block_means(k, block)
    return float(scale) * np.einsum("hud,hvd->huv", qb, kb)
