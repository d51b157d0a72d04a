"""Arithmetic facts the small-batch kernel's quantiser relies on, checked on the host.

The kernel forms the block scale sx = fp32(amax / 127) without a division, as
q0 = RN(amax * c), e = RN(amax - 127 q0) (one fma), sx = RN(e * c + q0) (one
fma), c = RN(1 / 127); and reads an int8 code straight from the low byte of
the fp32 bits of 1.5 * 2^23 + k.  Both are checked here exhaustively: the
first over every positive finite fp16 magnitude, the second over every code.
"""
from fractions import Fraction

import numpy as np

MAGIC = np.float32(12582912.0)  # 1.5 * 2^23


def rn32(x: Fraction) -> Fraction:
    """x rounded to the nearest binary32 value, ties to even (normal range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    assert e >= -126
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(x, ulp)
    if 2 * r > ulp or (2 * r == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def test_scale_without_division_equals_ieee_quotient():
    mags = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    ref = mags / np.float32(127.0)                     # IEEE binary32 division
    c = np.float32(1.0) / np.float32(127.0)
    q0 = mags * c                                      # RN(amax * c)
    # amax - 127 q0 is exact in binary64 (127 q0 has 31 significant bits and
    # the two terms are within a factor of two), so one conversion rounds once.
    e = (mags.astype(np.float64) - 127.0 * q0.astype(np.float64)).astype(np.float32)
    cf = Fraction(float(c))
    bad = []
    for i in range(mags.size):
        sx = rn32(Fraction(float(e[i])) * cf + Fraction(float(q0[i])))
        if sx != Fraction(float(ref[i])):
            bad.append(float(mags[i]))
    assert not bad, f"{len(bad)} magnitudes differ, first {bad[:5]}"


def test_magic_bits_hold_the_code():
    k = np.arange(-127, 128, dtype=np.int32)
    t = (MAGIC + k.astype(np.float32)).astype(np.float32)
    assert np.array_equal(t - MAGIC, k.astype(np.float32))
    low = (t.view(np.uint32) & 0xFF).astype(np.uint8).view(np.int8)
    assert np.array_equal(low.astype(np.int32), k)
