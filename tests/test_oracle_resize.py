"""Pins for the map-resize oracle (ScalingAttention section 4.3.1, Eq. 7)."""
import math

import numpy as np

from oracle.resize import bilinear, resize_region, resize_threshold


def test_bilinear_reproduces_linear_functions():
    """Bilinear interpolation is exact on a + b x + c y (inside the grid)."""
    n = 7
    xs = np.arange(n)
    R = 0.5 + 2.0 * xs[:, None] - 1.25 * xs[None, :]
    for nt in (7, 12, 20):
        for u in range(nt):
            for v in range(nt):
                x, y = u * n / nt, v * n / nt
                if x <= n - 1 and y <= n - 1:
                    assert abs(bilinear(R, u, v, nt) - (0.5 + 2.0 * x - 1.25 * y)) < 1e-12


def test_identity_when_sizes_match():
    rng = np.random.default_rng(1)
    keep = rng.random((2, 9, 9)) < 0.3
    assert np.array_equal(resize_region(keep, 9), keep)
    T = rng.random((2, 9, 9), dtype=np.float32)
    assert np.array_equal(resize_threshold(T, 9), T)


def _upscale2_rule(keep):
    """Integer rule for s = 2: target index t samples base t/2, or both neighbours of
    (t-1)/2 .. (t+1)/2 when t is odd (clamped at the last base index)."""
    H, n, _ = keep.shape
    out = np.zeros((H, 2 * n, 2 * n), bool)
    src = lambda t: [t // 2] if t % 2 == 0 else sorted({(t - 1) // 2, min((t + 1) // 2, n - 1)})
    for u in range(2 * n):
        for v in range(2 * n):
            out[:, u, v] = np.any([keep[:, a, b] for a in src(u) for b in src(v)], axis=0)
    return out


def test_upscale_by_two_closed_form():
    rng = np.random.default_rng(2)
    keep = rng.random((3, 6, 6)) < 0.25
    assert np.array_equal(resize_region(keep, 12), _upscale2_rule(keep))


def test_threshold_resize_commutes_with_thresholding():
    rng = np.random.default_rng(3)
    T = rng.random((2, 10, 10), dtype=np.float32)
    T[0, 2, 3] = np.nan
    for nt in (7, 10, 16, 23):
        Tt = resize_threshold(T, nt)
        for p in (0.1, 0.35, 0.6, 0.9):
            with np.errstate(invalid="ignore"):
                assert np.array_equal(resize_region(T <= p, nt), Tt <= p)


def test_region_resize_is_monotone_and_distributes_over_union():
    rng = np.random.default_rng(4)
    a = rng.random((1, 8, 8)) < 0.2
    b = rng.random((1, 8, 8)) < 0.2
    for nt in (5, 13):
        ra, rb, rab = resize_region(a, nt), resize_region(b, nt), resize_region(a | b, nt)
        assert np.array_equal(rab, ra | rb)
        assert np.all(rab >= ra)


def test_planted_floor_is_caught():
    keep = np.zeros((1, 4, 4), bool)
    keep[0, 1, 1] = True
    R = keep[0].astype(float)
    # target (3, 3) at s = 2 sits between base 1 and 2: ceil keeps it, floor would not
    assert math.ceil(bilinear(R, 3, 3, 8)) == 1 and math.floor(bilinear(R, 3, 3, 8)) == 0
    assert resize_region(keep, 8)[0, 3, 3]
