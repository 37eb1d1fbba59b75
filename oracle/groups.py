"""Adaptive per-output-channel group size (P1 §3.2, "Adaptive group quantization").

P1 gives sensitive channels more quantisation groups (finer) and robust ones
fewer, ranking them with an analytic sensitivity measure. That measure is not
given on the page; the reading used here is the first term of P1 eq. (3),
|W_ij| * ||X_j||_2, summed over the row of the pruned matrix, with the
column norms taken over a separate calibration batch:

    c_k = sqrt(sum_t Xcal[t, k]^2)            (sequential sum over t, FP64)
    S_n = sum_k |Wp[n, k]| * c_k              (sequential sum over k, FP64)

The ceil(frac * N) rows with the largest S_n (ties: lower n first) get the
fine group size, all others the coarse one. ``frac`` is taken to six decimal
places so that the count is an exact integer computation.
"""
import numpy as np


def column_norms(Xcal16: np.ndarray) -> np.ndarray:
    X = np.asarray(Xcal16, dtype=np.float16).astype(np.float64)
    return np.sqrt(np.cumsum(X * X, axis=0)[-1])


def sensitivity(W16: np.ndarray, mask: np.ndarray, Xcal16: np.ndarray) -> np.ndarray:
    W = np.asarray(W16, dtype=np.float16).astype(np.float64)
    Wp = np.where(mask, W, 0.0)
    c = column_norms(Xcal16)
    return np.cumsum(np.abs(Wp) * c[None, :], axis=1)[:, -1]


def fine_count(N: int, frac: float) -> int:
    """ceil(N * frac) with frac rounded to a multiple of 1e-6."""
    num = int(round(frac * 1_000_000))
    return (N * num + 999_999) // 1_000_000


def select_groups(W16, mask, Xcal16, frac=0.10, g_fine=32, g_coarse=128) -> np.ndarray:
    S = sensitivity(W16, mask, Xcal16)
    N = S.shape[0]
    order = np.argsort(-S, kind="stable")
    gs = np.full(N, g_coarse, dtype=np.int32)
    gs[order[: fine_count(N, frac)]] = g_fine
    return gs


def uniform_groups(N: int, g: int = 128) -> np.ndarray:
    return np.full(N, g, dtype=np.int32)
