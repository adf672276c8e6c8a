"""Hellinger distance and Fidelity Score between dense and sparse attention rows.

Pages: ScalingAttention section 4.2.1 -- the Hellinger distance of two discrete
distributions (Eq. 3) and the Fidelity Score F = 1 - H (Eq. 4) between a dense
attention distribution P and its sparse approximation P~; section 4.2.3 and
Appendix D, Table 6 -- the distance is estimated on a few rows drawn by
block-wise stratified sampling.

For a query row i of head h: P is softmax(scale * q_i K^T) over every key;
P~ is the softmax over the keys of the blocks the row's mask keeps, zero
elsewhere (the distribution sparse attention uses).

Readings used where the pages are silent: a row whose mask keeps nothing has
no P~; its distance is taken as 1 (the limit as the kept mass goes to 0);
the score of a head over sampled rows is 1 - mean of the row distances; the
sampled rows are an input (drawn elsewhere).

Computed in float64 from the given input values.  TEST INFRASTRUCTURE ONLY
(see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .crm import unpack_rows


def hellinger(p: np.ndarray, q: np.ndarray) -> float:
    """Eq. 3: (1/sqrt 2) * sqrt(sum_i (sqrt p_i - sqrt q_i)^2)."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return float(np.sqrt(np.sum((np.sqrt(p) - np.sqrt(q)) ** 2)) / np.sqrt(2.0))


def row_distributions(q_row, K, keep_keys, scale):
    """Dense P and sparse P~ (None when nothing is kept) for one query row."""
    s = scale * (np.asarray(K, np.float64) @ np.asarray(q_row, np.float64))
    e = np.exp(s - s.max())
    P = e / e.sum()
    if not keep_keys.any():
        return P, None
    sk = np.where(keep_keys, s, -np.inf)
    ek = np.exp(sk - sk[keep_keys].max())
    return P, ek / ek.sum()


def row_hellinger(Q, K, mask_bits, rows, scale, block=64):
    """Distance per sampled row: Q, K float arrays [H, N, d]; rows int [H, R]
    (token indices); returns float64 [H, R]."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    H, N, _ = Q.shape
    nb = -(-N // block)
    keep = unpack_rows(mask_bits, nb)                  # [H, nb, nb]
    out = np.zeros(np.asarray(rows).shape, np.float64)
    for h in range(H):
        for r, i in enumerate(np.asarray(rows)[h]):
            keys = np.repeat(keep[h, i // block], block)[:N]
            P, Pt = row_distributions(Q[h, i], K[h], keys, scale)
            out[h, r] = 1.0 if Pt is None else hellinger(P, Pt)
    return out


def head_fidelity(row_h: np.ndarray) -> np.ndarray:
    """Eq. 4 over the sampled rows of each head: 1 - mean row distance."""
    return 1.0 - np.asarray(row_h, np.float64).mean(axis=-1)
