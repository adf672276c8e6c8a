"""Checks on the seeded input generators (no method arithmetic lives there)."""
import numpy as np

import workloads


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38], np.float32)
    got = workloads.bf16_to_f32(workloads.bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties up to 1+2^-6
    assert got.tolist()[:5] == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5]
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000).astype(np.float32)
    r = workloads.bf16_to_f32(workloads.bf16_bits(y))
    assert np.max(np.abs(r - y) / np.abs(y)) <= 2**-8


def test_shapes_and_determinism():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.qkv(w)
    assert q.shape == (2, 256, 64) and q.dtype == np.float32
    q2, _, _ = workloads.qkv(w)
    assert np.array_equal(q, q2)
    _, k1, _ = workloads.qkv(w, heads=[1])
    assert np.array_equal(k1[0], k[1])
    m = workloads.masks(w)
    assert m.shape == (2, 4, 4) and m[:, np.arange(4), np.arange(4)].all()


def test_mask_densities_within_their_draw_ranges():
    w = workloads.WORKLOADS["wan13b_480p"]
    m = workloads.masks(w)
    dens = m.reshape(12, -1).mean(1)
    assert m.shape == (12, 512, 512)
    assert np.all(dens >= 0.099) and np.all(dens <= 0.501)
    nb = 512
    assert m[:, np.arange(nb), np.arange(nb)].all()
    w3 = workloads.WORKLOADS["wan14b_720p"]
    m3 = workloads.masks(w3)
    d3 = m3.reshape(40, -1).mean(1)
    assert int((d3 == 1.0).sum()) == 8
    assert np.all((d3 == 1.0) | ((d3 >= 0.0499) & (d3 <= 0.4001)))


def test_uniform_mask_exact_count():
    m = workloads.uniform_mask(3, 100, 0.2, seed=1)
    assert m.reshape(3, -1).sum(1).tolist() == [2000, 2000, 2000]
