"""Pins oracle.quant: hand-worked golden cases, grid-exact round trips, error bound."""
import numpy as np
import pytest

from oracle import quant
from conftest import read_golden


def test_hand_worked_golden():
    for rec in read_golden("quant_hand.txt"):
        v = np.array([float(t) for t in rec["v"].split()], dtype=np.float16)
        s16, z16, q = quant.quantize_groups(v[None, :])
        assert int(s16.view(np.uint16)[0]) == int(rec["s"], 16), rec
        assert int(z16.view(np.uint16)[0]) == int(np.float16(float(rec["z"])).view(np.uint16)), rec
        assert q[0].tolist() == [int(t) for t in rec["q"].split()], rec


@pytest.mark.parametrize("s", [2.0 ** -6, 2.0 ** -10, 3 * 2.0 ** -9, 5 * 2.0 ** -12])
def test_grid_exact_round_trip(s):
    rng = np.random.default_rng(int(s * 2 ** 20))
    G, m = 200, 16
    z = rng.integers(0, 16, G)
    q = rng.integers(0, 16, (G, m))
    q[:, 0], q[:, 1] = 0, 15                         # each group spans the full code range
    v = ((q - z[:, None]) * s).astype(np.float16)
    assert np.array_equal(v.astype(np.float64), (q - z[:, None]) * s)   # grid values are FP16-exact
    s16, z16, qq = quant.quantize_groups(v)
    assert np.all(s16.astype(np.float64) == s)
    assert np.array_equal(z16.astype(np.int64), z)
    assert np.array_equal(qq.astype(np.int64), q)
    assert np.array_equal(quant.dequantize(qq, s16, z16), v.astype(np.float64))


def test_half_step_bound_and_ranges():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((3000, 32)) * 0.02).astype(np.float16)
    s16, z16, q = quant.quantize_groups(v)
    s = s16.astype(np.float64)
    z = z16.astype(np.float64)
    assert np.all(s > 0) and np.all((z >= 0) & (z <= 15)) and np.all(z == np.rint(z))
    assert not np.any(np.signbit(z))                 # zero points are stored as +0, never -0
    assert q.max() <= 15
    wd = quant.dequantize(q, s16, z16)
    unclamped = (q > 0) & (q < 15)
    err = np.abs(wd - v.astype(np.float64))
    assert np.all(err[unclamped] <= s[:, None].repeat(32, 1)[unclamped] / 2)
    # the extremes are within one step even where clamping could act
    assert np.all(err <= s[:, None] * (1 + 1e-12))
    # zero is represented exactly (q == z dequantises to 0)
    assert np.all(quant.dequantize(np.broadcast_to(z[:, None], (3000, 1)).astype(np.uint8), s16, z16) == 0)
