"""Dense dequantise-then-dot reference in FP64 (P1 §1: INT4 weight-only GEMV).

The SparseGemv kernel computes y = W' x faster, where W' is the pruned,
quantised matrix dequantised back to real values; the plainest statement of
that result is the dense product, which is what this module computes.
"""
import numpy as np

from .fp16 import from_bits
from .pack import unpack_bytes


def dequant_dense(canon: dict) -> np.ndarray:
    """Canonical arrays -> dense W' (FP64 [N, K], zeros at pruned positions).
    FP16-valued arrays (key ``vals16``) hold the kept values themselves."""
    N, K, nk = canon["N"], canon["K"], canon["nk"]
    if "vals16" in canon:
        _, o = unpack_bytes(np.zeros((N, 1), np.uint8), canon["offs"])
        kpr = K * nk // 4
        j = np.arange(kpr, dtype=np.int64)
        col = 4 * (j[None, :] // nk) + o.astype(np.int64)
        Wd = np.zeros((N, K), dtype=np.float64)
        np.put_along_axis(Wd, col, from_bits(canon["vals16"]), axis=1)
        return Wd
    gs = np.asarray(canon["group_size"], dtype=np.int64)
    q, o = unpack_bytes(canon["vals"], canon["offs"])
    if nk == 4:                                   # dense: no stored offsets
        o = np.tile(np.arange(4, dtype=np.uint8), (N, K // 4))
    s = from_bits(canon["scale"])
    z = from_bits(canon["zero"])
    gptr = np.asarray(canon["gptr"], dtype=np.int64)
    kpr = K * nk // 4
    j = np.arange(kpr, dtype=np.int64)
    col = 4 * (j[None, :] // nk) + o.astype(np.int64)               # [N, kpr]
    grp = gptr[:N, None] + col // gs[:, None]                        # group of each element
    w = (q.astype(np.float64) - z[grp]) * s[grp]
    Wd = np.zeros((N, K), dtype=np.float64)
    np.put_along_axis(Wd, col, w, axis=1)
    return Wd


def gemv(Wd: np.ndarray, X16: np.ndarray) -> np.ndarray:
    """Y[b, n] = sum_k W'[n, k] * x[b, k] in FP64; X16 FP16 [B, K]."""
    X = np.asarray(X16, dtype=np.float16).astype(np.float64)
    return X @ Wd.T


def abs_dot(Wd: np.ndarray, X16: np.ndarray) -> np.ndarray:
    """D[b, n] = sum_k |W'[n, k] * x[b, k]|, the normaliser of the error."""
    X = np.asarray(X16, dtype=np.float16).astype(np.float64)
    return np.abs(X) @ np.abs(Wd).T


def normalized_error(y16: np.ndarray, y_ref: np.ndarray, D: np.ndarray) -> float:
    """max |y - y_ref| / D over all outputs; a zero D demands y == 0 exactly.

    y16 is the FP16 output widened exactly. Returns +inf when a D == 0 output
    is not zero, or when y holds a non-finite value.
    """
    y = np.asarray(y16, dtype=np.float16).astype(np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    diff = np.abs(y - y_ref)
    zero = D == 0
    if np.any(zero & (y != 0)):
        return float("inf")
    return float(np.max(np.where(zero, 0.0, diff / np.where(zero, 1.0, D)), initial=0.0))
