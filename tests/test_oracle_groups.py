"""Pins oracle.groups: exact rational sensitivities and the fine-row count."""
from fractions import Fraction

import numpy as np

from oracle import groups, prune


def test_exact_rational_ranking():
    # calibration columns with integer norms: (3,4)->5, (0,2)->2, (1,0)->1, (0,0)->0
    Xcal = np.array([[3, 0, 1, 0, 3, 0, 1, 0], [4, 2, 0, 0, 4, 2, 0, 0]], dtype=np.float16)
    c = [Fraction(5), Fraction(2), Fraction(1), Fraction(0)] * 2
    rng = np.random.default_rng(3)
    vals = np.array([0.0, 0.25, -0.5, 0.75, 1.0, -1.5, 2.0], dtype=np.float16)
    W = vals[rng.integers(0, len(vals), (9, 8))]
    offs, mask = prune.nm_prune(W, 2)
    S = groups.sensitivity(W, mask, Xcal)
    exact = []
    for n in range(9):
        s = sum(abs(Fraction(float(W[n, k]))) * c[k] for k in range(8) if mask[n, k])
        exact.append(s)
        assert S[n] == float(s)
    assert np.array_equal(groups.column_norms(Xcal), np.array([5, 2, 1, 0, 5, 2, 1, 0], dtype=float))
    for frac in (0.1, 0.3, 0.5):
        gs = groups.select_groups(W, mask, Xcal, frac, 32, 128)
        cnt = groups.fine_count(9, frac)
        # exact ranking: larger S first, lower n on ties
        order = sorted(range(9), key=lambda n: (-exact[n], n))
        assert sorted(np.nonzero(gs == 32)[0].tolist()) == sorted(order[:cnt])
        assert np.all((gs == 32) | (gs == 128))


def test_ties_prefer_lower_rows():
    W = np.ones((5, 8), dtype=np.float16)
    Xcal = np.ones((2, 8), dtype=np.float16)
    offs, mask = prune.nm_prune(W, 2)
    gs = groups.select_groups(W, mask, Xcal, 0.4, 32, 128)
    assert gs.tolist() == [32, 32, 128, 128, 128]


def test_fine_count():
    assert groups.fine_count(4096, 0.10) == 410
    assert groups.fine_count(11008, 0.10) == 1101
    assert groups.fine_count(30, 0.10) == 3          # 30*0.1 in FP64 is 3.0000000000000004
    assert groups.fine_count(10, 0.10) == 1
    assert groups.fine_count(1, 0.10) == 1
    assert groups.fine_count(100, 0.0) == 0
    assert groups.fine_count(100, 1.0) == 100
