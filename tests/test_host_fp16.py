"""The packer's FP64 -> FP16 conversion (sgemv_f64_to_f16, the routine that
rounds every group scale) against NumPy's float64 -> float16 cast, which is a
single round-to-nearest-even step (the oracle's FP16 pins show it against
exact rationals). CPU only: the library is loaded, no GPU call is made.

Cases: every one of the 65 536 half-precision values; every midpoint between
two consecutive halves, and the doubles just either side of it; 10^7 random
doubles spread over and beyond the FP16 range.
"""
import numpy as np

import sparse_weight_only_amd as sg


def numpy_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def test_every_half_round_trips():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = h.view(np.float16).astype(np.float64)
    out = sg.f64_to_f16(x)
    nan = np.isnan(x)
    assert np.array_equal(out[~nan], h[~nan])
    # NaN: the quiet NaN with the input's sign
    assert np.all(out[nan] == (0x7E00 | (h[nan] & 0x8000)))


def test_every_midpoint_ties_to_even():
    pos = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. 65504
    a = pos.view(np.float16).astype(np.float64)
    b = np.append(a[1:], 65536.0)                        # next half (65536 stands for +inf)
    mid = (a + b) / 2.0                                  # exact in FP64
    for sgn in (1.0, -1.0):
        m = sgn * mid
        got = sg.f64_to_f16(m)
        assert np.array_equal(got, numpy_bits(m))
        # a tie goes to the even neighbour: its last significand bit is 0
        assert np.all(got[np.abs(m) < 65504] & 1 == 0)
        for d in (np.inf, -np.inf):
            n = np.nextafter(m, d)
            assert np.array_equal(sg.f64_to_f16(n), numpy_bits(n))


def test_random_doubles():
    rng = np.random.default_rng(1234)
    total = 0
    for chunk in range(10):
        n = 1_000_000
        kind = chunk % 3
        if kind == 0:     # log-uniform magnitudes from 2^-30 to 2^20, both signs
            x = rng.standard_normal(n) * np.exp2(rng.uniform(-30, 20, n))
        elif kind == 1:   # random bit patterns with exponents around the FP16 range
            bits = rng.integers(0, 2 ** 52, n, dtype=np.uint64)
            e = rng.integers(1023 - 30, 1023 + 18, n).astype(np.uint64)
            sign = rng.integers(0, 2, n).astype(np.uint64)
            x = ((sign << np.uint64(63)) | (e << np.uint64(52)) | bits).view(np.float64)
        else:             # near the subnormal boundary and the overflow threshold
            x = np.concatenate([rng.uniform(-2.0 ** -13, 2.0 ** -13, n // 2),
                                rng.uniform(65000.0, 65600.0, n - n // 2) * rng.choice([-1, 1], n - n // 2)])
        assert np.array_equal(sg.f64_to_f16(x), numpy_bits(x)), f"chunk {chunk}"
        total += n
    assert total == 10_000_000


def test_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.999999, 65520.0, -65520.0,
                  2.0 ** -24, 2.0 ** -25, np.nextafter(2.0 ** -25, 1.0), 2.0 ** -26, 1e-300, -1e-300])
    assert np.array_equal(sg.f64_to_f16(x), numpy_bits(x))
    assert sg.f64_to_f16(np.array([np.nan]))[0] == 0x7E00
    assert sg.f64_to_f16(np.zeros(0)).size == 0
