"""Property tests over small random layers drawn by hypothesis.

* The oracle's N:M selection equals brute force over every kept subset of
  every group of 4, with values drawn from a small FP16 pool (+-0, repeated
  magnitudes) so that ties are frequent.
* The library's packer and layout equal the oracle's byte for byte on the
  same draws, for 2:4, 1:4 and the dense ablation, with a group size drawn
  per row (CPU only: the library is loaded, no GPU call).
"""
import numpy as np
import pytest
from hypothesis import given, settings, HealthCheck, strategies as st

import sparse_weight_only_amd as sg
from oracle import layout as olayout, pack as opack, prune as oprune
from test_oracle_prune import brute_kept

POOL = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 0.25, 3.0, -3.0, 6.1e-5, -6.0e-8, 65504.0 / 16],
                dtype=np.float16)


@st.composite
def layers(draw):
    N = draw(st.integers(1, 8))
    K = draw(st.sampled_from([256, 512]))
    nk = draw(st.sampled_from([1, 2, 4]))
    idx = draw(st.lists(st.integers(0, len(POOL) - 1), min_size=N * K, max_size=N * K))
    W = POOL[np.array(idx, dtype=np.int64)].reshape(N, K)
    gs = np.array(draw(st.lists(st.sampled_from([32, 64, 128, 256]), min_size=N, max_size=N)), np.int32)
    return W, nk, gs


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(layers())
def test_prune_is_brute_force_under_ties(layer):
    W, nk, _ = layer
    if nk == 4:
        return
    offs, mask = oprune.nm_prune(W, nk)
    N, K = W.shape
    for n in range(N):
        for j in range(K // 4):
            assert tuple(int(v) for v in offs[n, j]) == brute_kept(W[n, 4 * j: 4 * j + 4], nk)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(layers())
def test_library_pack_and_layout_equal_the_oracle(layer):
    W, nk, gs = layer
    N, K = W.shape
    co = opack.pack_canonical(W, nk, gs)
    cc = sg.pack(W, nk, gs)
    for k in ("vals", "offs", "scale", "zero", "gptr", "rowptr"):
        assert np.array_equal(cc[k], co[k]), k
    d = sg.describe(N, K, nk, gs)
    lay = olayout.build(co)
    try:
        blob = sg.layout(d, cc)
    except sg.SgemvError as e:
        # the layout refuses only groups whose FP16 dequantised values
        # would round past 65504 (values near the top of the FP16 range)
        assert e.code == sg.sgemv.SGEMV_EINVAL
        s = co["scale"].view(np.float16).astype(np.float64)
        z = co["zero"].view(np.float16).astype(np.float64)
        assert np.max(np.maximum(15 - z, z) * s) > 65504 - 16
        return
    assert np.array_equal(blob, lay["blob"])
