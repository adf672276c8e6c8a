"""Mask instantiation from a threshold map.

Pages: ScalingAttention, section 4.1.2 (Eq. 2 and the sentence after it) and
Appendix A, Algorithm 1 (phase 2, static block mask generation): each block
(u, v) of a head's threshold map T records the smallest sparsity level p at
which the block is active; a binary block mask for a target level p* is the
element-wise comparison M = I(T <= p*), one level per head (FAST selects
head-specific levels, section 4.2.2).

Reading used where the pages are silent: T and p* are float32 (the comparison
is exact in float32, so the mask is bit-exact); a NaN entry compares false and
is not kept; the comparison is inclusive (T == p* keeps the block).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .crm import pack_rows


def threshold_keep(T: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Boolean mask [H, n_q, n_k]: T[h, u, v] <= p[h], both float32."""
    T = np.asarray(T, dtype=np.float32)
    p = np.asarray(p, dtype=np.float32).reshape(-1)
    assert T.ndim == 3 and p.shape[0] == T.shape[0]
    with np.errstate(invalid="ignore"):
        return T <= p[:, None, None]


def threshold_mask_bits(T: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Packed row masks uint64 [H, n_q, ceil(n_k/64)] of threshold_keep."""
    return pack_rows(threshold_keep(T, p))
