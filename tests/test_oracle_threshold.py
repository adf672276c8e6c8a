"""Pins for the threshold-map mask oracle (ScalingAttention section 4.1.2, Eq. 2 and
the comparison after it; Appendix A, Algorithm 1, static block mask generation)."""
import json
import os

import numpy as np
import pytest

from oracle import crm
from oracle.threshold import threshold_keep, threshold_mask_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "threshold_hand_example.json")


def load_golden():
    g = json.load(open(GOLDEN))
    T = np.array([[[float(x) for x in row] for row in head] for head in g["T"]], dtype=np.float32)
    p = np.array(g["p"], dtype=np.float32)
    exp = np.array([[[int(w, 16) for w in row] for row in head] for head in g["expected_words"]],
                   dtype=np.uint64)
    return T, p, exp


def test_hand_example_words():
    T, p, exp = load_golden()
    assert np.array_equal(threshold_mask_bits(T, p), exp)


def test_tie_is_kept_and_nan_is_not():
    T = np.array([[[0.25, 0.5, np.nan, 0.75]]], dtype=np.float32)
    keep = threshold_keep(T, np.array([0.5], np.float32))
    assert keep.tolist() == [[[True, True, False, False]]]


def test_extreme_levels():
    rng = np.random.default_rng(3)
    T = rng.random((2, 5, 70), dtype=np.float32)
    T[0, 1, 2] = np.nan
    T[1, 0, 0] = -np.inf
    allk = threshold_keep(T, np.array([np.inf, np.inf], np.float32))
    assert allk.sum() == T.size - 1                       # everything but the NaN
    nonek = threshold_keep(T, np.array([-np.inf, -np.inf], np.float32))
    assert nonek.sum() == 1 and nonek[1, 0, 0]            # only the -inf entry


def test_monotone_in_level_and_per_head():
    rng = np.random.default_rng(4)
    T = rng.random((3, 6, 130), dtype=np.float32)
    levels = np.linspace(0, 1, 11, dtype=np.float32)
    prev = None
    for lv in levels:
        k = threshold_keep(T, np.full(3, lv, np.float32))
        if prev is not None:
            assert np.all(k >= prev)
        prev = k
    # each head uses its own level
    k = threshold_keep(T, np.array([0.0, 0.5, 1.0], np.float32))
    assert not k[0].any() or np.all(T[0][k[0]] <= 0)
    assert k[2].all()
    assert np.array_equal(k[1], T[1] <= np.float32(0.5))


def test_packing_round_trip():
    rng = np.random.default_rng(5)
    T = rng.random((2, 4, 200), dtype=np.float32)
    p = np.array([0.3, 0.7], np.float32)
    bits = threshold_mask_bits(T, p)
    assert bits.shape == (2, 4, crm.words_per_row(200 * 64, 64))
    assert np.array_equal(crm.unpack_rows(bits, 200), threshold_keep(T, p))


def test_planted_strict_comparison_is_caught():
    """A strict '<' in place of '<=' must fail the hand example (the tie at v = 70)."""
    T, p, exp = load_golden()
    wrong = crm.pack_rows(T < p[:, None, None])
    assert not np.array_equal(wrong, exp)
