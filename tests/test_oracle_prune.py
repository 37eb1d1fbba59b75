"""Pins oracle.prune: brute force over every kept subset of every group of 4."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import prune


def brute_kept(group, nk):
    """Kept set = max sum of |w|; among equal sums the lexicographically smallest columns."""
    best = None
    for sub in itertools.combinations(range(4), nk):
        key = (sum(Fraction(abs(float(group[p]))) for p in sub), tuple(-p for p in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return best[1]


@pytest.mark.parametrize("nk", [1, 2])
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_with_forced_ties(nk, seed):
    rng = np.random.default_rng(seed)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, 0.25, -1.0], dtype=np.float16)
    W = pool[rng.integers(0, len(pool), (7, 64))] if seed % 2 == 0 else \
        (rng.standard_normal((7, 64)) * 0.02).astype(np.float16)
    offs, mask = prune.nm_prune(W, nk)
    assert offs.shape == (7, 16, nk) and mask.sum() == 7 * 16 * nk
    for n in range(7):
        for j in range(16):
            g = W[n, 4 * j: 4 * j + 4]
            want = brute_kept(g, nk)
            assert tuple(int(v) for v in offs[n, j]) == want
            kept = np.abs(g[list(want)].astype(np.float64))
            dropped = np.abs(np.delete(g, list(want)).astype(np.float64))
            assert kept.min() >= dropped.max()


def test_offsets_ascending_and_values():
    W = np.array([[0.1, -0.3, 0.2, 0.0, 4.0, 3.0, 2.0, 1.0]], dtype=np.float16)
    offs, mask = prune.nm_prune(W, 2)
    assert offs.tolist() == [[[1, 2], [0, 1]]]
    assert prune.kept_values(W, offs).astype(np.float64).tolist() == \
        [[float(np.float16(-0.3)), float(np.float16(0.2)), 4.0, 3.0]]
    assert prune.kept_columns(offs).tolist() == [[1, 2, 4, 5]]
    offs1, _ = prune.nm_prune(W, 1)
    assert offs1.tolist() == [[[1], [0]]]


def test_all_equal_keeps_lowest_columns():
    W = np.full((2, 8), 0.5, dtype=np.float16)
    W[1, :] = [-0.0, 0.0, -0.0, 0.0, 1, -1, 1, -1]
    offs, _ = prune.nm_prune(W, 2)
    assert offs.tolist() == [[[0, 1], [0, 1]], [[0, 1], [0, 1]]]


def test_rejects_non_finite():
    W = np.zeros((1, 8), dtype=np.float16)
    W[0, 3] = np.inf
    with pytest.raises(ValueError):
        prune.nm_prune(W, 2)
