"""Pins for the Hellinger / Fidelity oracle (ScalingAttention Eqs. 3-4, sections
4.2.1 and 4.2.3)."""
import math

import numpy as np

import workloads
from oracle import crm
from oracle.fidelity import head_fidelity, hellinger, row_distributions, row_hellinger


def test_hellinger_textbook_cases():
    assert hellinger([0.2, 0.3, 0.5], [0.2, 0.3, 0.5]) == 0.0
    assert abs(hellinger([1, 0, 0], [0, 0.5, 0.5]) - 1.0) < 1e-15        # disjoint supports
    # two Bernoulli laws: H^2 = 1 - (sqrt(ab) + sqrt((1-a)(1-b)))  (Bhattacharyya form)
    for a, b in ((0.1, 0.7), (0.5, 0.5), (0.01, 0.99)):
        ref = math.sqrt(1 - (math.sqrt(a * b) + math.sqrt((1 - a) * (1 - b))))
        assert abs(hellinger([a, 1 - a], [b, 1 - b]) - ref) < 1e-15
    p, q = [0.1, 0.6, 0.3], [0.5, 0.25, 0.25]
    assert hellinger(p, q) == hellinger(q, p)


def test_restriction_closed_form():
    """P~ is P restricted to the kept keys and renormalised, so the distance depends
    only on the kept dense mass rho: H = sqrt(1 - sqrt(rho))."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        n = int(rng.integers(2, 300))
        K = rng.standard_normal((n, 16))
        q = rng.standard_normal(16)
        keep = rng.random(n) < rng.uniform(0.05, 0.95)
        keep[rng.integers(n)] = True
        P, Pt = row_distributions(q, K, keep, 0.7)
        rho = P[keep].sum()
        assert abs(hellinger(P, Pt) - math.sqrt(max(0.0, 1 - math.sqrt(rho)))) < 1e-12


def test_full_mask_is_exact_and_supersets_never_increase_distance():
    rng = np.random.default_rng(2)
    H, N, d = 2, 300, 16
    Q = rng.standard_normal((H, N, d)); K = rng.standard_normal((H, N, d))
    nb = -(-N // 64)
    rows = workloads.stratified_rows(H, N, 8, seed=3)
    full = crm.pack_rows(np.ones((H, nb, nb), bool))
    assert np.all(row_hellinger(Q, K, full, rows, 0.25) < 1e-7)
    keep = rng.random((H, nb, nb)) < 0.3
    more = keep | (rng.random((H, nb, nb)) < 0.3)
    h1 = row_hellinger(Q, K, crm.pack_rows(keep), rows, 0.25)
    h2 = row_hellinger(Q, K, crm.pack_rows(more), rows, 0.25)
    assert np.all(h2 <= h1 + 1e-12)
    assert np.all((h1 >= 0) & (h1 <= 1))


def test_empty_row_reading_and_head_score():
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((1, 128, 8)); K = rng.standard_normal((1, 128, 8))
    keep = np.zeros((1, 2, 2), bool); keep[0, 1, 1] = True
    rows = np.array([[5, 100]], np.int32)                # row block 0 keeps nothing
    h = row_hellinger(Q, K, crm.pack_rows(keep), rows, 0.5)
    assert h[0, 0] == 1.0 and 0 < h[0, 1] < 1
    assert abs(head_fidelity(h)[0] - (1 - (1.0 + h[0, 1]) / 2)) < 1e-15


def test_stratified_rows_one_per_stratum():
    rows = workloads.stratified_rows(3, 75600, 16, seed=9)
    edges = (np.arange(17) * 75600) // 16
    for h in range(3):
        for r in range(16):
            assert edges[r] <= rows[h, r] < edges[r + 1]


def test_planted_missing_factor_is_caught():
    """Dropping Eq. 3's 1/sqrt(2) gives sqrt(2) on disjoint supports, not the bound 1."""
    wrong = lambda p, q: float(np.sqrt(np.sum((np.sqrt(p) - np.sqrt(q)) ** 2)))
    assert abs(wrong([1, 0], [0, 1]) - 1.0) > 0.4
    assert abs(hellinger([1, 0], [0, 1]) - 1.0) < 1e-15
