"""Seeded synthetic inputs for the SparseGemv workloads.

This module only draws random numbers and casts them to FP16. It holds none
of the method's arithmetic (no pruning, grouping, quantisation, packing or
products), so both the oracle side (``oracle/``) and the HIP side
(``sparse_weight_only_amd``) can be fed from it without sharing any code.

Recipe (the pages train on proprietary ad data that is not available; these
seeded layers stand in for it):

* every array comes from ``numpy.random.default_rng(SeedSequence([seed, cfg,
  layer, mat, tag]))`` with tag 0 = weights, 1 = activations,
  2 = calibration batch, 3 = outlier channel choice;
* weights: ``fp16(0.02 * standard_normal((N, K)))``, row n = output channel;
* activations: ``fp16(standard_normal((B, K)))``; the 4096x4096 workload
  additionally multiplies ``round(0.01*K)`` channels (drawn without
  replacement) by 20 in FP64 before the FP16 cast;
* calibration batch for the adaptive group choice: T = 64 rows drawn like x.

All FP16 casts are NumPy's round-to-nearest-even conversion from FP64.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

TAG_W, TAG_X, TAG_XCAL, TAG_OUTLIER = 0, 1, 2, 3
LLAMA7B_MATS: Tuple[Tuple[str, int, int], ...] = (
    # (name, K in, N out) of one LLaMA-7B-shaped decoder layer
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 11008),
    ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
)


def rng(cfg: int, layer: int = 0, mat: int = 0, tag: int = 0, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, layer, mat, tag]))


def weights(N: int, K: int, cfg: int, layer: int = 0, mat: int = 0, seed: int = 0,
            std: float = 0.02) -> np.ndarray:
    """FP16 N x K weight matrix ~ N(0, std^2), C order."""
    g = rng(cfg, layer, mat, TAG_W, seed)
    return (std * g.standard_normal((N, K))).astype(np.float16)


def activations(B: int, K: int, cfg: int, layer: int = 0, mat: int = 0, seed: int = 0,
                outlier_frac: float = 0.0, outlier_scale: float = 20.0) -> np.ndarray:
    """FP16 B x K activations ~ N(0, 1); optional outlier channels scaled in FP64."""
    g = rng(cfg, layer, mat, TAG_X, seed)
    x = g.standard_normal((B, K))
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        idx = rng(cfg, layer, mat, TAG_OUTLIER, seed).choice(K, size=n_out, replace=False)
        x[:, idx] *= outlier_scale
    return x.astype(np.float16)


def calibration(T: int, K: int, cfg: int, layer: int = 0, mat: int = 0, seed: int = 0) -> np.ndarray:
    """FP16 T x K calibration batch used only to rank output channels."""
    g = rng(cfg, layer, mat, TAG_XCAL, seed)
    return g.standard_normal((T, K)).astype(np.float16)


@dataclasses.dataclass(frozen=True)
class Layer:
    """One GEMV of a workload: shapes, N:M choice, group policy and seeds."""
    name: str
    K: int
    N: int
    nk: int                 # kept per group of 4 along K (2 -> 2:4, 1 -> 1:4)
    adaptive: bool          # True: top 10% rows by sensitivity use g=32, rest g=128
    w_cfg: int              # seed coordinates of the weights
    layer: int
    mat: int
    x_cfg: int
    outlier_frac: float = 0.0

    def W(self, seed: int = 0) -> np.ndarray:
        return weights(self.N, self.K, self.w_cfg, self.layer, self.mat, seed)

    def X(self, B: int = 1, seed: int = 0) -> np.ndarray:
        return activations(B, self.K, self.x_cfg, self.layer, self.mat, seed, self.outlier_frac)

    def Xcal(self, T: int = 64, seed: int = 0) -> np.ndarray:
        return calibration(T, self.K, self.w_cfg, self.layer, self.mat, seed)


FRAC_FINE, G_FINE, G_COARSE, CALIB_T = 0.10, 32, 128, 64


def cfg1() -> List[Layer]:
    """Single 1024 -> 1024 layer, 2:4, uniform g=128, batch 1."""
    return [Layer("cfg1_1024x1024_2of4", 1024, 1024, 2, False, 1, 0, 0, 1)]


def cfg2() -> List[Layer]:
    """4096 -> 4096 attention projection, 2:4, uniform g=128, 1% outlier channels x20."""
    return [Layer("cfg2_4096x4096_2of4", 4096, 4096, 2, False, 2, 0, 0, 2, outlier_frac=0.01)]


def cfg3() -> List[Layer]:
    """MLP up (4096 -> 11008) and down (11008 -> 4096), each at 1:4 and at 2:4, adaptive groups."""
    out = []
    for nk in (1, 2):
        tag = "1of4" if nk == 1 else "2of4"
        out.append(Layer(f"cfg3_up_4096x11008_{tag}", 4096, 11008, nk, True, 3, nk, 5, 3))
        out.append(Layer(f"cfg3_down_11008x4096_{tag}", 11008, 4096, nk, True, 3, nk, 6, 3))
    return out


def layer_nk(layer: int, n_layers: int = 32) -> int:
    """Layer-wise N:M policy of the 32-layer set: 2:4 for the first and last 4 layers."""
    return 2 if (layer < 4 or layer >= n_layers - 4) else 1


def cfg4(n_layers: int = 32) -> List[Layer]:
    """All 7 projections of a 32-layer 7B-shaped decoder (224 GEMVs)."""
    out = []
    for l in range(n_layers):
        nk = layer_nk(l, n_layers)
        for m, (name, K, N) in enumerate(LLAMA7B_MATS):
            out.append(Layer(f"cfg4_l{l:02d}_{name}", K, N, nk, True, 4, l, m, 4))
    return out


def cfg5() -> List[Layer]:
    """Beam-batch shapes: up/down of layer 0 (2:4) and layer 4 (1:4) of the 32-layer set."""
    out = []
    for l in (0, 4):
        nk = layer_nk(l)
        for m in (5, 6):
            name, K, N = LLAMA7B_MATS[m]
            out.append(Layer(f"cfg5_l{l:02d}_{name}", K, N, nk, True, 4, l, m, 5))
    return out


CFG5_BATCHES = (4, 8, 16)
