"""3D Hilbert-curve token order.

DFSAttn abstract (listed on the PSA page and the SPADE page): tokens are
reordered along a Hilbert curve so that tokens close in (frame, height, width)
land in the same block.  The pages name the curve but not its construction;
this uses J. Skilling's transpose construction ("Programming the Hilbert
curve", AIP Conf. Proc. 707, 2004) on the smallest 2^b cube holding the grid,
axes ordered (t, y, x), with the index read off the transposed coordinates
most significant bit first.  The permutation lists token ids (t-major
flattening t*H*W + y*W + x) in increasing curve index; indices are distinct,
so no ties arise.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def hilbert_index(coords: np.ndarray, bits: int) -> np.ndarray:
    """Curve index of integer points coords [P, n] with 0 <= coords < 2^bits."""
    x = np.array(coords, dtype=np.int64, copy=True)
    n = x.shape[1]
    # undo excess work: walk the bit levels from the top, inverting the low bits
    # of axis 0 or swapping low bits between axis 0 and axis i
    q = 1 << (bits - 1)
    while q > 1:
        low = q - 1
        for i in range(n):
            hi = (x[:, i] & q) != 0
            x[hi, 0] ^= low
            swap = (x[~hi, 0] ^ x[~hi, i]) & low
            x[~hi, 0] ^= swap
            x[~hi, i] ^= swap
        q >>= 1
    # Gray encode across axes
    for i in range(1, n):
        x[:, i] ^= x[:, i - 1]
    t = np.zeros(x.shape[0], np.int64)
    q = 1 << (bits - 1)
    while q > 1:
        t ^= np.where((x[:, n - 1] & q) != 0, q - 1, 0)
        q >>= 1
    x ^= t[:, None]
    # interleave: bit level b (high to low), axis 0 first
    idx = np.zeros(x.shape[0], np.int64)
    for b in range(bits - 1, -1, -1):
        for i in range(n):
            idx = (idx << 1) | ((x[:, i] >> b) & 1)
    return idx


def grid_bits(T: int, H: int, W: int) -> int:
    m = max(T, H, W)
    return max(1, int(m - 1).bit_length())


def hilbert_order(T: int, H: int, W: int) -> np.ndarray:
    """int32 permutation: entry i is the token id at position i along the curve."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    pts = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)
    idx = hilbert_index(pts, grid_bits(T, H, W))
    return np.argsort(idx, kind="stable").astype(np.int32)


def permute_rows(x: np.ndarray, perm: np.ndarray, inverse: bool = False) -> np.ndarray:
    """y[:, i] = x[:, perm[i]] (gather), or y[:, perm[i]] = x[:, i] (inverse)."""
    perm = np.asarray(perm)
    if not inverse:
        return x[:, perm]
    y = np.empty_like(x)
    y[:, perm] = x
    return y
