"""Semi-structured N:M pruning along K (P1 §3.2, "Sparsification").

P1 prunes each layer with an N:M pattern, 2:4 for the important layers and
1:4 for the others, keeping the elements with the highest importance. The
importance of eq. (3) needs activation norms and loss gradients; with no
model or data, the score here is the weight magnitude |w| (the first term of
eq. (3) with unit activation norms). Groups are 4 consecutive input columns
of one output row. Exactly ``nk`` elements are kept per group, ties going to
the lower column; the kept offsets are stored in ascending order.
"""
import numpy as np


def nm_prune(W16: np.ndarray, nk: int):
    """Select the kept elements of every group of 4 along K.

    W16: FP16 [N, K] (row = output channel), K % 4 == 0; nk in {1, 2}, or 4
         for the dense (unpruned) ablation, which keeps every element.
    Returns (offs, mask):
      offs: uint8 [N, K//4, nk]  in-group column offsets of the kept
            elements, ascending;
      mask: bool [N, K] True where the element is kept.
    """
    W = np.asarray(W16, dtype=np.float16)
    N, K = W.shape
    if K % 4 or nk not in (1, 2, 4):
        raise ValueError("K must be a multiple of 4 and nk in {1, 2, 4}")
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    a = np.abs(W.astype(np.float64)).reshape(N, K // 4, 4)
    # rank by |w| descending; a stable sort keeps equal magnitudes in column
    # order, so the lower column wins a tie (and -0 ties +0)
    order = np.argsort(-a, axis=-1, kind="stable")
    offs = np.sort(order[..., :nk], axis=-1).astype(np.uint8)
    mask = np.zeros((N, K // 4, 4), dtype=bool)
    np.put_along_axis(mask, offs.astype(np.int64), True, axis=-1)
    return offs, mask.reshape(N, K)


def kept_values(W16: np.ndarray, offs: np.ndarray) -> np.ndarray:
    """FP16 values of the kept elements, [N, K*nk/4], ascending column order."""
    W = np.asarray(W16, dtype=np.float16)
    N, K = W.shape
    nk = offs.shape[-1]
    v = np.take_along_axis(W.reshape(N, K // 4, 4), offs.astype(np.int64), axis=-1)
    return v.reshape(N, K // 4 * nk)


def kept_columns(offs: np.ndarray) -> np.ndarray:
    """Column index of every kept element, [N, K*nk/4]: 4*group + offset."""
    N, G, nk = offs.shape
    base = (4 * np.arange(G, dtype=np.int64))[None, :, None]
    return (base + offs.astype(np.int64)).reshape(N, G * nk)


def column_scale(Xcal16, K: int) -> np.ndarray:
    """c_k = sqrt(sum_t Xcal[t, k]^2) (sequential sum over t, FP64); all ones
    when no calibration batch is given."""
    if Xcal16 is None:
        return np.ones(K, dtype=np.float64)
    X = np.asarray(Xcal16, dtype=np.float16).astype(np.float64)
    if X.ndim != 2 or X.shape[1] != K or X.shape[0] < 1:
        raise ValueError("calibration batch must be [T, K] with T >= 1")
    if not np.all(np.isfinite(X)):
        raise ValueError("non-finite activation")
    return np.sqrt(np.cumsum(X * X, axis=0)[-1])


def nm_prune_scored(W16: np.ndarray, nk: int, Xcal16=None):
    """N:M selection by the activation-aware importance of P1 §3.2, eq. (3),
    first term: score(n, k) = |W[n, k]| * ||X[:, k]||_2, the column norm taken
    over a calibration batch (the gradient term needs a loss and a trained
    model and is left out). Per group of 4 along K the nk largest scores are
    kept (FP64 products; ties to the lower column), offsets ascending.
    Without a calibration batch the score is |w| and this is ``nm_prune``.

    Returns (offs, mask) like ``nm_prune``.
    """
    W = np.asarray(W16, dtype=np.float16)
    N, K = W.shape
    if K % 4 or nk not in (1, 2):
        raise ValueError("K must be a multiple of 4 and nk in {1, 2}")
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    c = column_scale(Xcal16, K)
    score = (np.abs(W.astype(np.float64)) * c[None, :]).reshape(N, K // 4, 4)
    order = np.argsort(-score, axis=-1, kind="stable")
    offs = np.sort(order[..., :nk], axis=-1).astype(np.uint8)
    mask = np.zeros((N, K // 4, 4), dtype=bool)
    np.put_along_axis(mask, offs.astype(np.int64), True, axis=-1)
    return offs, mask.reshape(N, K)


def pruned_dense(W16: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """FP16 [N, K]: the kept values (bits unchanged) and +0 at pruned positions."""
    W = np.asarray(W16, dtype=np.float16)
    return np.where(mask, W, np.float16(0.0)).astype(np.float16)
