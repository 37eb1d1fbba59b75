"""Pins oracle.fp16 against an exact rational round-to-nearest-even (IEEE 754 binary16)."""
from fractions import Fraction

import numpy as np

from oracle import fp16


def exact_rne_fp16_bits(x: float) -> int:
    """IEEE 754 binary16 RNE of a finite double, computed with exact rationals."""
    f = Fraction(x)
    sign = 0x8000 if (f < 0 or (f == 0 and np.signbit(x))) else 0
    a = abs(f)
    if a >= Fraction(65520):                       # 65504 + half ulp, tie -> even (overflow)
        return sign | 0x7C00
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                                # subnormals share quantum 2^-24
    quantum = Fraction(2) ** (e - 10)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum                              # may carry into the next binade
    if val >= Fraction(65520) or val > Fraction(65504):
        return sign | 0x7C00
    if val < Fraction(2) ** -14:
        return sign | int(val / Fraction(2) ** -24)
    E = val.numerator.bit_length() - val.denominator.bit_length()
    while Fraction(2) ** E > val:
        E -= 1
    while Fraction(2) ** (E + 1) <= val:
        E += 1
    mant = int(val / Fraction(2) ** (E - 10)) - 1024
    return sign | ((E + 15) << 10) | mant


def test_all_halves_round_trip():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = u.view(np.float16)
    fin = np.isfinite(h)
    back = fp16.bits(fp16.to_fp16(h[fin].astype(np.float64)))
    assert np.array_equal(back, u[fin])


def test_midpoints_and_neighbours_match_exact_rounding():
    u = np.arange(0, 0x7BFF, dtype=np.uint16)          # positive finite, each with a successor
    a = u.view(np.float16).astype(np.float64)
    b = (u + 1).view(np.float16).astype(np.float64)
    mid = (a + b) / 2                                    # exact in FP64
    rng = np.random.default_rng(7)
    pick = rng.choice(len(mid), size=3000, replace=False)
    for m in mid[pick]:
        for x in (m, np.nextafter(m, -np.inf), np.nextafter(m, np.inf), -m):
            assert int(fp16.bits(fp16.to_fp16(x))) == exact_rne_fp16_bits(float(x)), x
    # every midpoint: ties go to the even neighbour
    got = fp16.bits(fp16.to_fp16(mid))
    even = np.where(u % 2 == 0, u, u + 1).astype(np.uint16)
    assert np.array_equal(got, even)


def test_random_doubles_match_exact_rounding():
    rng = np.random.default_rng(11)
    xs = rng.standard_normal(4000) * np.exp2(rng.integers(-30, 17, 4000))
    for x in xs:
        assert int(fp16.bits(fp16.to_fp16(x))) == exact_rne_fp16_bits(float(x)), x


def test_overflow_and_subnormal_edges():
    for x, want in [(65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (2.0 ** -24, 0x0001),
                    (2.0 ** -25, 0x0000), (2.0 ** -25 * 1.0000001, 0x0001), (3 * 2.0 ** -25, 0x0002),
                    (2.0 ** -14, 0x0400), (-0.0, 0x8000)]:
        assert int(fp16.bits(fp16.to_fp16(x))) == want == exact_rne_fp16_bits(x), x
