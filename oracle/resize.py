"""Resolution scaling of block maps (ScalingAttention section 4.3.1, Eq. 7).

The page resizes a base-resolution map to a target block count by bilinear
interpolation at (u / s, v / s) followed by a ceiling, so that any overlap with
an active region survives.  Readings used (the printed rule is ambiguous; see the
design notes):

* Eq. 7 is applied to a binary region map R (1 = active block): the target
  value is ceil(bilinear(R, u / s, v / s)) with s = n_target / n_base for both
  axes (the map is square: query blocks x key blocks), base samples at integer
  coordinates 0 .. n_base - 1, coordinates past the last sample clamped to it.
  A ceiling of a value in [0, 1] is 1 exactly when some sample with positive
  interpolation weight is active.
* For a threshold map the ceiling would not be conservative (a larger threshold
  means less activity), so its counterpart is the minimum over the samples with
  positive weight: a target block is then active at level p exactly when the
  resized region map of I(T <= p) says so.  NaN entries are ignored by the
  minimum (they are never active).

Plain float64 bilinear arithmetic.  TEST INFRASTRUCTURE ONLY (see the package
docstring).
"""
from __future__ import annotations

import math

import numpy as np


def _axis(u: int, n_base: int, n_target: int):
    """Bilinear sample indices and weights along one axis at x = u / s."""
    x = u * n_base / n_target
    x0 = min(int(math.floor(x)), n_base - 1)
    fx = min(max(x - x0, 0.0), 1.0) if x0 < n_base - 1 else 0.0
    x1 = min(x0 + 1, n_base - 1)
    return x0, x1, fx


def bilinear(R: np.ndarray, u: int, v: int, n_target: int) -> float:
    n = R.shape[-1]
    x0, x1, fx = _axis(u, n, n_target)
    y0, y1, fy = _axis(v, n, n_target)
    return ((1 - fx) * (1 - fy) * R[x0, y0] + fx * (1 - fy) * R[x1, y0]
            + (1 - fx) * fy * R[x0, y1] + fx * fy * R[x1, y1])


def resize_region(keep: np.ndarray, n_target: int) -> np.ndarray:
    """Eq. 7 on boolean maps [H, n_base, n_base] -> [H, n_target, n_target]."""
    keep = np.asarray(keep, bool)
    H = keep.shape[0]
    out = np.zeros((H, n_target, n_target), bool)
    R = keep.astype(np.float64)
    for h in range(H):
        for u in range(n_target):
            for v in range(n_target):
                out[h, u, v] = math.ceil(bilinear(R[h], u, v, n_target)) >= 1
    return out


def resize_threshold(T: np.ndarray, n_target: int) -> np.ndarray:
    """Conservative resize of float32 threshold maps: min over positive-weight samples."""
    T = np.asarray(T, np.float32)
    H, n, _ = T.shape
    out = np.empty((H, n_target, n_target), np.float32)
    for h in range(H):
        for u in range(n_target):
            x0, x1, fx = _axis(u, n, n_target)
            xs = [x0] + ([x1] if fx > 0 else [])
            for v in range(n_target):
                y0, y1, fy = _axis(v, n, n_target)
                ys = [y0] + ([y1] if fy > 0 else [])
                out[h, u, v] = np.fmin.reduce(np.array([T[h, a, b] for a in xs for b in ys], np.float32))
    return out
