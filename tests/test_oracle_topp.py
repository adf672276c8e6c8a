"""Pins for the float32 top-p selection procedure and its exponential."""
import math

import numpy as np
import pytest

import workloads
from oracle import topp

F = np.float32


def test_exp32_accuracy_against_libm():
    xs = np.concatenate([np.linspace(-87.0, 0.0, 20001), -np.logspace(-8, 1.9, 3000)]).astype(F)
    got = topp.exp32(xs).astype(np.float64)
    want = np.array([math.exp(float(x)) for x in xs])
    rel = np.abs(got - want) / want
    assert rel.max() < 4e-7          # a few float32 ulps


def test_exp32_special_values():
    assert topp.exp32(np.array([0.0], F))[0] == F(1.0)
    assert topp.exp32(np.array([-88.0, -np.inf], F)).tolist() == [0.0, 0.0]
    assert topp.exp32(np.array([-1.0], F))[0] == pytest.approx(math.exp(-1.0), rel=2e-7)


def test_float32_cumsum_is_sequential():
    rng = np.random.default_rng(1)
    x = rng.random(3000).astype(F) * F(1e-3)
    acc = F(0.0)
    seq = []
    for v in x:
        acc = F(acc + v)
        seq.append(acc)
    assert np.array_equal(np.cumsum(x, dtype=F), np.array(seq, F))


def test_tiny_p_keeps_exactly_the_top_min_blocks():
    s = workloads.random_scores(2, 5, 300, seed=2)
    keep = topp.topp_keep(s, 1e-30, 8)
    for h in range(2):
        for u in range(5):
            want = np.argsort(-s[h, u].astype(np.float64), kind="stable")[:8]
            assert set(np.flatnonzero(keep[h, u]).tolist()) == set(want.tolist())


def test_kept_sets_nest_as_p_grows():
    s = workloads.random_scores(1, 6, 200, seed=3)
    prev = None
    for p in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):
        k = topp.topp_keep(s, p, 8)
        if prev is not None:
            assert np.all(k >= prev)
        prev = k


def test_equal_scores_keep_a_lowest_index_prefix():
    s = np.zeros((1, 1, 50), F)
    keep = topp.topp_keep(s, 0.5, 8)[0, 0]
    k = int(keep.sum())
    assert keep[:k].all() and not keep[k:].any()
    assert k == 25           # 25 equal shares of 1/50 reach one half


def test_one_dominant_score_keeps_min_blocks():
    s = np.zeros((1, 1, 100), F)
    s[0, 0, 37] = 50.0
    keep = topp.topp_keep(s, 0.9, 8)[0, 0]
    assert keep.sum() == 8 and keep[37] and keep[:7].all()


def test_short_rows_keep_everything():
    s = workloads.random_scores(1, 3, 5, seed=4)
    assert topp.topp_keep(s, 0.5, 8).all()


def test_agrees_with_float64_except_on_boundary_rows():
    s = workloads.random_scores(2, 40, 400, seed=5, spread=2.0)
    keep = topp.topp_keep(s, 0.9, 8)
    disagree = 0
    for h in range(2):
        for u in range(40):
            row = s[h, u].astype(np.float64)
            order = np.argsort(-row, kind="stable")
            c = np.cumsum(np.exp(row[order] - row.max()))
            c /= c[-1]
            k = max(int(np.argmax(c >= 0.9)) + 1, 8)
            ref = np.zeros(400, bool)
            ref[order[:k]] = True
            if not np.array_equal(ref, keep[h, u]):
                disagree += 1
                assert topp.boundary_margin(row, 0.9, 8) < 1e-5
    assert disagree <= 2


def test_selection_mass_reaches_p():
    s = workloads.random_scores(1, 20, 300, seed=6)
    keep = topp.topp_keep(s, 0.9, 8)
    for u in range(20):
        row = s[0, u].astype(np.float64)
        pr = np.exp(row - row.max()); pr /= pr.sum()
        kept_mass = pr[keep[0, u]].sum()
        assert kept_mass >= 0.9 - 1e-5
        # dropping the smallest kept block falls below p (unless min-k binds)
        if keep[0, u].sum() > 8:
            assert kept_mass - pr[keep[0, u]].min() < 0.9 + 1e-5


def test_all_nan_row_reads_as_equal_scores():
    """A row of NaN scores clamps to a row of equal scores: equal shares, so the
    lowest-index prefix that reaches p (25 of 50 at p = 1/2), as for equal scores."""
    s = np.full((1, 1, 50), np.nan, F)
    keep = topp.topp_keep(s, 0.5, 0)[0, 0]
    assert keep[:25].all() and not keep[25:].any()


def test_positive_infinity_takes_all_mass():
    """One +inf among finite scores: every other exponential underflows to 0 against
    it, so k_p = 1 and the top-k minimum adds the 7 best finite blocks (score
    descending, lower index first on ties)."""
    s = workloads.random_scores(1, 1, 300, seed=8)
    s[0, 0, 123] = np.inf
    s[0, 0, 7] = s[0, 0, 9]                      # a tie among the finite scores
    keep = topp.topp_keep(s, 0.9, 8)[0, 0]
    others = np.array([j for j in np.argsort(-s[0, 0].astype(np.float64), kind="stable") if j != 123])
    want = np.zeros(300, bool)
    want[123] = True
    want[others[:7]] = True
    assert np.array_equal(keep, want)
    assert topp.topp_keep(s, 0.9, 1)[0, 0].sum() == 1


def test_nan_and_negative_infinity_rank_below_every_finite_score():
    """NaN and -inf both read as -FLT_MAX: they are kept only once every finite block
    is, and then in index order.  (An oracle without the clamp keeps the whole row,
    since a NaN maximum makes every sum NaN.)"""
    rng = np.random.default_rng(9)
    s = (rng.standard_normal(30) * 3).astype(F)
    idx = rng.permutation(30)
    s[idx[:5]] = np.nan
    s[idx[5:10]] = -np.inf
    finite = np.sort(idx[10:])
    low = np.sort(idx[:10])
    keep = topp.topp_keep(s[None, None], 1e-6, 20)[0, 0]
    assert np.array_equal(np.flatnonzero(keep), finite)
    keep = topp.topp_keep(s[None, None], 1e-6, 22)[0, 0]
    assert np.array_equal(np.flatnonzero(keep), np.sort(np.concatenate([finite, low[:2]])))
    # the mass of p is carried by the finite blocks alone
    fin = s[finite].astype(np.float64)
    pr = np.exp(fin - fin.max())
    pr /= pr.sum()
    kept = topp.topp_keep(s[None, None], 0.9, 0)[0, 0]
    assert not kept[low].any() and pr[np.isin(finite, np.flatnonzero(kept))].sum() >= 0.9 - 1e-6
