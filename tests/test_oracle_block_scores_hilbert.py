"""Pins for the block-score oracle and the Hilbert order."""
import math

import numpy as np

from oracle import block_scores, hilbert


def test_constant_blocks_closed_form():
    H, nb, d = 2, 4, 8
    rng = np.random.default_rng(1)
    a = rng.standard_normal((H, nb, d))
    b = rng.standard_normal((H, nb, d))
    n = nb * 64 - 30
    q = np.repeat(a, 64, axis=1)[:, :n]
    k = np.repeat(b, 64, axis=1)[:, :n]
    s = block_scores.block_scores(q, k, 0.125)
    for h in range(H):
        for u in range(nb):
            for v in range(nb):
                want = 0.125 * math.fsum(a[h, u, c] * b[h, v, c] for c in range(d))
                assert abs(s[h, u, v] - want) <= 1e-13


def test_tail_block_averages_only_real_tokens():
    n = 64 + 1
    x = np.zeros((1, n, 3))
    x[0, 64] = [3.0, -1.0, 2.0]
    x[0, :64] = 1.0
    m = block_scores.block_means(x)
    assert np.array_equal(m[0, 1], [3.0, -1.0, 2.0])
    assert np.array_equal(m[0, 0], [1.0, 1.0, 1.0])


def test_brute_force_small():
    rng = np.random.default_rng(2)
    n, d = 150, 4
    q = rng.standard_normal((1, n, d)); k = rng.standard_normal((1, n, d))
    s = block_scores.block_scores(q, k, 0.5)
    blocks = [list(range(b * 64, min(n, b * 64 + 64))) for b in range(3)]
    for u in range(3):
        for v in range(3):
            qm = [math.fsum(q[0, i, c] for i in blocks[u]) / len(blocks[u]) for c in range(d)]
            km = [math.fsum(k[0, j, c] for j in blocks[v]) / len(blocks[v]) for c in range(d)]
            assert abs(s[0, u, v] - 0.5 * math.fsum(x * y for x, y in zip(qm, km))) <= 1e-13


def test_hilbert_full_cube_is_a_unit_step_bijection():
    """Every cube up to 2^7 (the cube that holds the 21 x 45 x 80 latent grid):
    the index is a bijection onto [0, 8^b), consecutive indices are unit steps
    on one axis, and each run of 8^(b-1) consecutive indices fills one octant
    (the recursive structure of a Hilbert curve)."""
    for bits in range(1, 8):
        side = 1 << bits
        g = np.stack(np.meshgrid(*[np.arange(side)] * 3, indexing="ij"), -1).reshape(-1, 3)
        idx = hilbert.hilbert_index(g, bits)
        assert np.array_equal(np.sort(idx), np.arange(side ** 3))
        path = g[np.argsort(idx)]
        steps = np.abs(np.diff(path, axis=0)).sum(axis=1)
        assert np.all(steps == 1)
        octant = (path >> (bits - 1)).reshape(8, -1, 3)
        assert np.all(octant == octant[:, :1])
        assert len({tuple(o) for o in octant[:, 0]}) == 8
    assert hilbert.grid_bits(21, 45, 80) == 7


def test_hilbert_2d_unit_steps():
    for bits in (1, 2, 4):
        side = 1 << bits
        g = np.stack(np.meshgrid(np.arange(side), np.arange(side), indexing="ij"), -1).reshape(-1, 2)
        path = g[np.argsort(hilbert.hilbert_index(g, bits))]
        assert np.all(np.abs(np.diff(path, axis=0)).sum(axis=1) == 1)


def test_hilbert_order_is_a_permutation_and_local():
    perm = hilbert.hilbert_order(21, 45, 80)
    assert perm.dtype == np.int32 and perm.size == 75600
    assert np.array_equal(np.sort(perm), np.arange(75600))
    # tokens sharing a 64-token block along the curve stay close in (t, y, x)
    t, r = np.divmod(perm.astype(np.int64), 45 * 80)
    y, x = np.divmod(r, 80)
    span = []
    for b in range(0, 75600, 64):
        sl = slice(b, b + 64)
        span.append((np.ptp(t[sl]), np.ptp(y[sl]), np.ptp(x[sl])))
    span = np.array(span)
    assert np.median(span.max(axis=1)) <= 8


def test_permute_roundtrip():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 50, 4))
    perm = rng.permutation(50).astype(np.int32)
    y = hilbert.permute_rows(x, perm)
    assert np.array_equal(y[:, 3], x[:, perm[3]])
    assert np.array_equal(hilbert.permute_rows(y, perm, inverse=True), x)
