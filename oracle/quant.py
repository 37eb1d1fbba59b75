"""Asymmetric INT4 group quantisation of the kept weights.

P1 §1 ("our core idea") compresses FP16 weights to INT4 for a weight-only
GEMV, with group-wise quantisation whose group count adapts per channel
(P1 §3.2). The page gives no formula; the reading used is plain min-max
asymmetric quantisation with FP16 scale and zero per group:

* a group of row n covers ``g`` consecutive dense columns; only the kept
  elements of those columns (g*nk/4 values, ascending column) are quantised;
* lo = min(0, min v), hi = max(0, max v)  (zero is always representable;
  a -0 minimum counts as 0);
* hi == lo (all kept values zero): scale 1, zero 0, every code 0;
* otherwise scale = fp16((hi - lo) / 15) computed in FP64 and rounded once to
  FP16, raised to 2^-24 if it underflows to 0;
* zero = clamp(rint(-lo / scale), 0, 15), an integer held as FP16 (+0, never
  -0, when it is zero);
* code = clamp(rint(v / scale) + zero, 0, 15)  (rint before adding zero);
* dequantised weight = (code - zero) * scale, exact in FP64 and in FP32.

All rint are round-half-to-even.
"""
import numpy as np

from .fp16 import to_fp16

S_MIN = 2.0 ** -24


def quantize_groups(v16: np.ndarray):
    """Quantise a batch of groups.

    v16: FP16 [G, m] kept values of G groups (m values each).
    Returns (scale16 FP16 [G], zero16 FP16 [G], q uint8 [G, m]).
    """
    v = np.asarray(v16, dtype=np.float16).astype(np.float64)
    G = v.shape[0]
    vmin, vmax = v.min(axis=1), v.max(axis=1)
    lo = np.where(vmin < 0.0, vmin, 0.0)
    hi = np.where(vmax > 0.0, vmax, 0.0)
    flat = hi == lo
    t = (hi - lo) / 15.0
    s16 = to_fp16(np.where(flat, 1.0, t))
    s16 = np.where(s16.astype(np.float64) < S_MIN, np.float16(S_MIN), s16).astype(np.float16)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-lo / s), 0.0, 15.0)
    z = np.where(flat, 0.0, z) + 0.0          # +0.0 turns a -0 zero point into +0
    q = np.clip(np.rint(v / s[:, None]) + z[:, None], 0.0, 15.0)
    q = np.where(flat[:, None], 0.0, q)
    return s16, z.astype(np.float16), q.astype(np.uint8)


def dequantize(q: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """(q - zero) * scale in FP64; q [G, m], scale/zero [G]."""
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)
    z = np.asarray(zero16, dtype=np.float16).astype(np.float64)
    return (q.astype(np.float64) - z[:, None]) * s[:, None]
