"""Pins for the stripe-mask oracle (PSA page, Figure 3 and Appendix Tables 7-9)."""
import json
import os

import numpy as np

import workloads
from oracle import crm, stripes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _one_axis_distances(n, w, o, s):
    a = np.arange(n)
    d = a[None, :] - a[:, None]
    keep = stripes.in_stripe(d, w, o, s)
    return sorted(set(d[keep].tolist()))


def test_hand_worked_examples():
    g = json.load(open(os.path.join(GOLD, "stripe_hand_example.json")))
    assert _one_axis_distances(g["n"], g["width"], g["offset"], g["gap"]) == g["kept_distances"]
    assert _one_axis_distances(g["n2"], g["width2"], g["offset2"], g["gap2"]) == g["kept_distances2"]
    assert _one_axis_distances(g["n3"], g["width3"], g["offset3"], g["gap3"]) == g["kept_distances3"]


def test_full_window_is_all_ones():
    p = np.array([[1, 1, 0, 0, 1, 0, 0]], np.int32)
    keep = stripes.stripe_keep(p, 5, 4 * 64, 5 * 4 * 64)
    assert keep.all()


def test_unit_widths_give_exactly_the_block_diagonal():
    p = np.array([[0, 1, 0, 0, 1, 0, 0]], np.int32)
    T, fb = 6, 5
    keep = stripes.stripe_keep(p, T, fb * 64, T * fb * 64)
    assert np.array_equal(keep[0], np.eye(T * fb, dtype=bool))


def _band_pairs(n, w):
    """Closed form: pairs (a, b) in [0,n)^2 whose distance lies in the band
    [-floor(w/2), w-1-floor(w/2)] -- sum over distances of (n - |d|)."""
    lo, hi = -(w // 2), w - 1 - w // 2
    return sum(n - abs(d) for d in range(lo, hi + 1) if abs(d) < n)


def test_single_band_counts_closed_form():
    # Tw = 5 over 33 frames: 33 + 2*32 + 2*31 frame pairs
    assert _band_pairs(33, 5) == 159
    for n, w in [(33, 5), (21, 7), (9, 1), (60, 10), (7, 3)]:
        assert stripes.stripe_count_1d(n, w, 0, 0) == _band_pairs(n, w)


def test_aligned_frames_factorise_into_axis_counts():
    rng = np.random.default_rng(11)
    T, fb = 7, 6
    for _ in range(12):
        tw = int(rng.choice([1, 3, 5, 7])); sw = int(rng.choice([1, 3, 5, 10]))
        ss = int(rng.choice([0, 1, 3, 6]))
        p = np.array([[0, tw, 0, 0, sw, 0, ss]], np.int32)
        keep = stripes.stripe_keep(p, T, fb * 64, T * fb * 64)[0]
        # closed-form temporal count (single band) times the spatial count
        # enumerated directly from the kept-distance set
        sp = stripes.stripe_count_1d(fb, sw, 0, ss)
        assert keep.sum() == _band_pairs(T, tw) * sp


def test_symmetry_for_odd_widths_zero_offset():
    for tw, sw, ss in [(5, 3, 3), (7, 1, 6), (1, 5, 1)]:
        p = np.array([[0, tw, 0, 0, sw, 0, ss]], np.int32)
        keep = stripes.stripe_keep(p, 5, 6 * 64, 5 * 6 * 64)[0]
        assert np.array_equal(keep, keep.T)


def test_printed_tuples_give_distinct_masks():
    """Under the gap reading every printed tuple yields its own mask; under a
    'stride = period' reading pairs such as (3,0,3) and (3,0,1) would coincide."""
    g = json.load(open(os.path.join(GOLD, "psa_stripe_tuples.json")))
    w = workloads.WORKLOADS["hunyuan_768"]
    T, F = 33, 60 * 64
    for name, rows in g["tables"].items():
        seen = set()
        for t in rows:
            p = np.array([[0] + list(t)], np.int32)
            bits = stripes.stripe_mask_bits(p, T, F, T * F)
            key = bits.tobytes()
            assert key not in seen, (name, t)
            seen.add(key)
    assert g["full_window_share_percent"] == [20.0, 20.0, 20.0]


def test_wider_band_contains_narrower():
    for a, b in [(1, 5), (5, 7), (3, 11)]:
        pa = np.array([[0, a, 0, 0, 3, 0, 3]], np.int32)
        pb = np.array([[0, b, 0, 0, 3, 0, 3]], np.int32)
        ka = stripes.stripe_keep(pa, 12, 4 * 64, 12 * 4 * 64)
        kb = stripes.stripe_keep(pb, 12, 4 * 64, 12 * 4 * 64)
        assert np.all(kb >= ka)


def test_unaligned_frames_use_first_token_placement():
    # frame of 100 tokens: block 3 starts at token 192 -> frame 1, spatial block (92 // 64) = 1
    t, s = stripes.block_coords(5, 100, 64)
    assert t.tolist() == [0, 0, 1, 1, 2] and s.tolist() == [0, 1, 0, 1, 0]


def test_hunyuan_workload_density_band():
    w = workloads.WORKLOADS["hunyuan_768"]
    params = workloads.stripe_params(w)
    assert params.shape == (24, 7) and int(params[:, 0].sum()) == 5
    for p in params:
        if p[0]:
            continue
        cnt = stripes.stripe_count_1d(33, p[1], p[2], p[3]) * stripes.stripe_count_1d(60, p[4], p[5], p[6])
        dens = cnt / 1980.0 ** 2
        assert 0.003 < dens < 0.2
    bits = stripes.stripe_mask_bits(params[:3], 33, 3840, w.seq_len)
    assert bits.shape == (3, 1980, 31)
    assert crm.unpack_rows(bits, 1980).sum() == stripes.stripe_keep(params[:3], 33, 3840, w.seq_len).sum()
