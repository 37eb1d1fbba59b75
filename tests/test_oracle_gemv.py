"""Pins oracle.gemv: exact rational sums, an independent element-by-element decode."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemv, pack


def decode_triplets(c):
    """Independent decode of the canonical arrays into (row, column, value) triplets."""
    N, K, nk = c["N"], c["K"], c["nk"]
    out = []
    for n in range(N):
        g = int(c["group_size"][n])
        for j in range(K * nk // 4):
            code = (int(c["vals"][n, j // 2]) >> (4 * (j % 2))) & 0xF
            if nk == 4:                          # dense ablation: element j is column j
                col = j
            else:
                off = (int(c["offs"][n, j // 4]) >> (2 * (j % 4))) & 3
                col = 4 * (j // nk) + off
            gi = int(c["gptr"][n]) + col // g
            s = float(np.uint16(c["scale"][gi]).view(np.float16))
            z = float(np.uint16(c["zero"][gi]).view(np.float16))
            out.append((n, col, Fraction(code) - Fraction(z), Fraction(s)))
    return out


@pytest.mark.parametrize("nk", [1, 2, 4])
def test_exact_rational_gemv(nk):
    rng = np.random.default_rng(10 + nk)
    N, K, B = 6, 256, 3
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    gs = np.array([32, 128, 128, 32, 128, 64], dtype=np.int32)
    c = pack.pack_canonical(W, nk, gs)
    X = rng.standard_normal((B, K)).astype(np.float16)
    Wd = gemv.dequant_dense(c)
    Y = gemv.gemv(Wd, X)
    D = gemv.abs_dot(Wd, X)
    trip = decode_triplets(c)
    assert np.count_nonzero(Wd) <= len(trip) == N * K * nk // 4
    for b in range(B):
        ex = [Fraction(0)] * N
        ab = [Fraction(0)] * N
        fs = [[] for _ in range(N)]
        for (n, col, qz, s) in trip:
            t = qz * s * Fraction(float(X[b, col]))
            ex[n] += t
            ab[n] += abs(t)
            fs[n].append(float(t))
            assert Wd[n, col] == float(qz * s)                 # FP64 dequantisation is exact
        for n in range(N):
            assert abs(Y[b, n] - float(ex[n])) <= 1e-14 * float(ab[n]) + 1e-300
            assert abs(D[b, n] - float(ab[n])) <= 1e-14 * float(ab[n]) + 1e-300
            assert abs(math.fsum(fs[n]) - Y[b, n]) <= 1e-14 * float(ab[n]) + 1e-300


def test_unit_vectors_and_ones():
    rng = np.random.default_rng(2)
    N, K = 9, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    c = pack.pack_canonical(W, 2, [128] * N)
    Wd = gemv.dequant_dense(c)
    for k in (0, 1, 255, 511):
        e = np.zeros((1, K), dtype=np.float16)
        e[0, k] = 1
        assert np.array_equal(gemv.gemv(Wd, e)[0], Wd[:, k])
    ones = np.ones((1, K), dtype=np.float16)
    assert np.allclose(gemv.gemv(Wd, ones)[0], [math.fsum(r) for r in Wd], rtol=1e-14, atol=0)
    # exactly nk non-zeros at most per group of 4, none at pruned positions
    mask = c["mask"]
    assert np.all(Wd[~mask] == 0)


def test_normalized_error_rules():
    y_ref = np.array([[1.0, 0.0, -2.0]])
    D = np.array([[2.0, 0.0, 4.0]])
    assert gemv.normalized_error(np.array([[1.0, 0.0, -2.0]], dtype=np.float16), y_ref, D) == 0.0
    assert gemv.normalized_error(np.array([[1.5, 0.0, -2.0]], dtype=np.float16), y_ref, D) == 0.25
    assert gemv.normalized_error(np.array([[1.0, 2 ** -24, -2.0]], dtype=np.float16), y_ref, D) == float("inf")
    assert gemv.normalized_error(np.array([[np.nan, 0.0, -2.0]], dtype=np.float16), y_ref, D) == float("inf")
