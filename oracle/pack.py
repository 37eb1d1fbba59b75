"""Canonical index-compressed "2bit-CSR" arrays (P1 §1, contributions, first item).

P1 replaces the column indices of CSR by a compressed index for mixed 2:4 /
1:4 sparsity and states that index plus weights shrink to 30 % of plain CSR.
The page gives no bit layout; the reading used here (one that reproduces the
30 % exactly: 4-bit value + 2-bit offset = 6 bits against 4-bit value + 16-bit
column index = 20 bits) is, for row n and its kept element j (ascending
column, j = 0 .. K*nk/4 - 1, column 4*(j // nk) + off_j):

* vals  uint8 [N, K*nk/8]   code of element j in byte j//2, low nibble if j even;
* offs  uint8 [N, K*nk/16]  off_j in byte j//4, bits 2*(j%4) .. 2*(j%4)+1;
* scale, zero  uint16 [n_groups]  FP16 bit patterns, row-major over (n, group);
* gptr  int32 [N+1]  first group of row n (the ragged row pointer of the
  scale/zero arrays: sum over earlier rows of K/g_m);
* rowptr int32 [N+1] first kept element of row n (n*K*nk/4; regular because
  every group of 4 keeps exactly nk elements).

nk = 4 is the dense INT4 ablation (the plain weight-only GEMV that
SparseGemv extends, P1 §1 contributions, second item): every element is
kept, element j is column j, and no offsets are stored (``offs`` has zero
bytes per row).
"""
import numpy as np

from . import prune as _prune
from . import quant as _quant
from .fp16 import bits


def sizes(N: int, K: int, nk: int, group_size) -> dict:
    gs = np.asarray(group_size, dtype=np.int64)
    kept = N * K * nk // 4
    return {
        "kept": kept,
        "vals_bytes": kept // 2,
        "offs_bytes": 0 if nk == 4 else kept // 4,
        "n_groups": int(np.sum(K // gs)),
    }


def quantize_rows(kept16: np.ndarray, nk: int, K: int, group_size: np.ndarray):
    """Quantise every row with its own group size; returns per-row groups in row order."""
    N = kept16.shape[0]
    gs = np.asarray(group_size, dtype=np.int64)
    q = np.zeros(kept16.shape, dtype=np.uint8)
    ng = K // gs
    gptr = np.zeros(N + 1, dtype=np.int64)
    gptr[1:] = np.cumsum(ng)
    scale = np.zeros(int(gptr[-1]), dtype=np.float16)
    zero = np.zeros(int(gptr[-1]), dtype=np.float16)
    for g in np.unique(gs):
        rows = np.nonzero(gs == g)[0]
        m = int(g) * nk // 4
        v = kept16[rows].reshape(len(rows) * (K // int(g)), m)
        s16, z16, qq = _quant.quantize_groups(v)
        q[rows] = qq.reshape(len(rows), -1)
        idx = (gptr[rows][:, None] + np.arange(K // int(g))[None, :]).reshape(-1)
        scale[idx] = s16
        zero[idx] = z16
    return q, scale, zero, gptr


def pack_bytes(q: np.ndarray, o: np.ndarray):
    """Per-element codes/offsets [N, kpr] -> canonical vals/offs bytes."""
    N, kpr = q.shape
    q = q.astype(np.uint16)
    o = o.astype(np.uint16)
    vals = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    offs = (o[:, 0::4] | (o[:, 1::4] << 2) | (o[:, 2::4] << 4) | (o[:, 3::4] << 6)).astype(np.uint8)
    return vals, offs


def unpack_bytes(vals: np.ndarray, offs: np.ndarray):
    """Inverse of pack_bytes: canonical bytes -> per-element codes and offsets."""
    N = vals.shape[0]
    q = np.empty((N, vals.shape[1] * 2), dtype=np.uint8)
    q[:, 0::2] = vals & 0xF
    q[:, 1::2] = vals >> 4
    o = np.empty((N, offs.shape[1] * 4), dtype=np.uint8)
    for i in range(4):
        o[:, i::4] = (offs >> (2 * i)) & 3
    return q, o


def pack_canonical(W16: np.ndarray, nk: int, group_size) -> dict:
    """Dense FP16 W -> prune -> quantise -> canonical 2bit-CSR arrays."""
    W = np.asarray(W16, dtype=np.float16)
    N, K = W.shape
    gs = np.asarray(group_size, dtype=np.int64)
    if gs.shape != (N,) or np.any(gs % 32) or np.any(K % gs) or K % 256:
        raise ValueError("bad shape or group sizes")
    offs3, mask = _prune.nm_prune(W, nk)
    kept16 = _prune.kept_values(W, offs3)
    q, scale, zero, gptr = quantize_rows(kept16, nk, K, gs)
    o = offs3.reshape(N, -1)
    vals, offs = pack_bytes(q, o)
    if nk == 4:
        offs = np.zeros((N, 0), dtype=np.uint8)      # dense: column j is element j
    kpr = K * nk // 4
    return {
        "N": N, "K": K, "nk": nk, "group_size": gs.astype(np.int32),
        "vals": vals, "offs": offs,
        "scale": bits(scale), "zero": bits(zero),
        "gptr": gptr.astype(np.int32),
        "rowptr": (np.arange(N + 1, dtype=np.int64) * kpr).astype(np.int32),
        "mask": mask,
    }


def pack_fp16_canonical(W16: np.ndarray, nk: int) -> dict:
    """FP16-valued 2bit-CSR (P1 §1 "our core idea" and contributions, first
    item: semi-structured layer-wise FP16 mixed sparsity, before INT4): the
    same N:M selection and 2-bit offsets, the kept values stored as FP16.

    * vals16 uint16 [N, K*nk/4]  FP16 bits of kept element j (ascending column);
    * offs   uint8  [N, K*nk/16] as in the INT4 form;
    * rowptr int32  [N+1]        n*K*nk/4.
    """
    W = np.asarray(W16, dtype=np.float16)
    N, K = W.shape
    if K % 256 or nk not in (1, 2):
        raise ValueError("K must be a multiple of 256 and nk in {1, 2}")
    offs3, mask = _prune.nm_prune(W, nk)
    kept16 = _prune.kept_values(W, offs3)
    _, offs = pack_bytes(np.zeros(kept16.shape, np.uint8), offs3.reshape(N, -1))
    kpr = K * nk // 4
    return {"N": N, "K": K, "nk": nk, "vals16": bits(kept16), "offs": offs,
            "rowptr": (np.arange(N + 1, dtype=np.int64) * kpr).astype(np.int32), "mask": mask}
