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


# ---- activation-aware score |w| * ||x_k|| (eq. (3), first term)

def brute_kept_scored(scores, nk):
    """Same rule on exact scores: max sum; among equal sums the lowest columns."""
    best = None
    for sub in itertools.combinations(range(4), nk):
        key = (sum(scores[p] for p in sub), tuple(-p for p in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return best[1]


def test_scored_hand_worked_group():
    # w = 1/2, 1/4, 1/8, 1/16 and one calibration row x = 1/8, 1, 1, 8:
    # column norms 1/8, 1, 1, 8 and scores 1/16, 1/4, 1/8, 1/2. By |w| the
    # first two columns win; by score columns 3 then 1.
    W = np.array([[0.5, 0.25, 0.125, 0.0625]], dtype=np.float16)
    X = np.array([[0.125, 1.0, 1.0, 8.0]], dtype=np.float16)
    assert prune.nm_prune_scored(W, 2, X)[0].tolist() == [[[1, 3]]]
    assert prune.nm_prune_scored(W, 1, X)[0].tolist() == [[[3]]]
    assert prune.nm_prune(W, 2)[0].tolist() == [[[0, 1]]]
    # two calibration rows: norms sqrt(1/64 + 1/64), sqrt(2), sqrt(2), sqrt(128)
    X2 = np.vstack([X, X])
    assert prune.nm_prune_scored(W, 2, X2)[0].tolist() == [[[1, 3]]]
    # a zero column scale drops its weight whatever its size
    Xz = np.array([[0.0, 1.0, 1.0, 1.0]], dtype=np.float16)
    assert prune.nm_prune_scored(np.array([[9.0, 0.25, 0.125, 0.0625]], np.float16), 1, Xz)[0].tolist() == [[[1]]]
    dense = prune.pruned_dense(W, prune.nm_prune_scored(W, 2, X)[1])
    assert dense.tolist() == [[0.0, 0.25, 0.0, 0.0625]]


@pytest.mark.parametrize("nk", [1, 2])
@pytest.mark.parametrize("seed", range(6))
def test_scored_brute_force_exact(nk, seed):
    """One calibration row makes c_k = |x_k| exactly, and |w| * |x| of two FP16
    magnitudes is exact in FP64, so exact rational scores decide."""
    rng = np.random.default_rng(100 + seed)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, 0.25, -2.0], dtype=np.float16)
    if seed % 2 == 0:
        W = pool[rng.integers(0, len(pool), (5, 64))]
        X = pool[rng.integers(0, len(pool), (1, 64))]
    else:
        W = (rng.standard_normal((5, 64)) * 0.02).astype(np.float16)
        X = rng.standard_normal((1, 64)).astype(np.float16)
    offs, mask = prune.nm_prune_scored(W, nk, X)
    assert mask.sum() == 5 * 16 * nk
    for n in range(5):
        for j in range(16):
            sc = [Fraction(abs(float(W[n, 4 * j + p]))) * Fraction(abs(float(X[0, 4 * j + p]))) for p in range(4)]
            assert tuple(int(v) for v in offs[n, j]) == brute_kept_scored(sc, nk)


def test_scored_reduces_to_magnitude():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((6, 256)) * 0.02).astype(np.float16)
    for nk in (1, 2):
        ref = prune.nm_prune(W, nk)[0]
        assert np.array_equal(prune.nm_prune_scored(W, nk, None)[0], ref)
        const = np.full((3, 256), -0.75, dtype=np.float16)          # equal column norms
        assert np.array_equal(prune.nm_prune_scored(W, nk, const)[0], ref)
