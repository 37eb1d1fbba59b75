"""FP64 <-> FP16 conversion for the oracle.

FP16 scale and zero per group are fixed by the weight-only INT4 scheme of P1
§1 ("our core idea": compress FP16 weights to INT4). The conversion is a
single round-to-nearest-even from FP64 (no detour through FP32), which is
what NumPy's ``astype(float16)`` does; tests pin it against exact rational
rounding.
"""
import numpy as np


def to_fp16(a) -> np.ndarray:
    """Round FP64 values to FP16 (nearest, ties to even)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16)


def bits(h: np.ndarray) -> np.ndarray:
    """FP16 array -> uint16 bit patterns."""
    return np.asarray(h, dtype=np.float16).view(np.uint16)


def from_bits(u: np.ndarray) -> np.ndarray:
    """uint16 bit patterns -> FP64 values (exact)."""
    return np.asarray(u, dtype=np.uint16).view(np.float16).astype(np.float64)
