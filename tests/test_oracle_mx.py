"""Pins of the MX oracle (oracle/mx.py) against the OCP MX v1.0 definitions: element
tables, brute-force rounding, the shared-exponent rule, exact power-of-two scaling and
the lossless special case that reduces the product to a plain matmul."""
import math

import numpy as np
import pytest

from oracle import mx

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the specification's FP4 E2M1 values


def test_e2m1_table_and_sign():
    assert mx.e2m1_value(np.arange(8)).tolist() == E2M1_TABLE
    assert mx.e2m1_value(np.arange(8, 16)).tolist() == [-v for v in E2M1_TABLE]


def test_e4m3_landmarks():
    v = mx.e4m3_value
    assert v(0x00) == 0.0
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x38) == 1.0                # bias 7
    assert v(0x7E) == 448.0              # largest normal
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x80 | 0x38) == -1.0
    mags = v(np.arange(0x7F))
    assert np.all(np.diff(mags) > 0)     # monotone in the code


def _brute_round(values, table, max_code):
    """Nearest representable magnitude by exhaustive search, ties to the even code."""
    out = []
    for x in values:
        a = min(abs(x), table[max_code])
        d = [abs(a - t) for t in table[: max_code + 1]]
        best = min(d)
        cands = [c for c, dd in enumerate(d) if dd == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(c | ((0x80 if max_code == 0x7E else 0x8) if (x < 0 and c != 0) else 0))
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_rounding_matches_brute_force(fmt):
    if fmt == "e4m3":
        table, max_code, rnd = mx.e4m3_value(np.arange(0x7F)).tolist(), 0x7E, mx.round_e4m3
    else:
        table, max_code, rnd = E2M1_TABLE, 0x7, mx.round_e2m1
    g = np.random.default_rng(1)
    mids = [(a + b) / 2 for a, b in zip(table[:max_code], table[1:max_code + 1])]
    vals = (list(table) + mids + [-m for m in mids] +
            list(g.uniform(-1.2, 1.2, 300) * table[max_code]) +
            list(g.uniform(-1, 1, 200) * table[3]) + [table[max_code] * 1.7, -1e6])
    assert np.array_equal(rnd(np.array(vals)), _brute_round(vals, table, max_code))


@pytest.mark.parametrize("fmt,emax", [("e4m3", 8), ("e2m1", 2)])
def test_shared_exponent_rule(fmt, emax):
    g = np.random.default_rng(2)
    x = (g.standard_normal((6, 128)) * np.exp2(g.integers(-12, 12, size=(6, 1)))).astype(np.float16)
    codes, scales = mx.mx_quantize(x, fmt)
    for r in range(6):
        for b in range(4):
            amax = float(np.max(np.abs(x[r, 32 * b:32 * b + 32].astype(np.float64))))
            e = math.frexp(amax)[1] - 1                       # floor(log2 amax)
            assert int(scales[r, b]) == e - emax + 127
            # the largest element lands in the top binade [2^emax, 2^(emax+1)), saturated to max
            big = np.argmax(np.abs(x[r, 32 * b:32 * b + 32].astype(np.float64)))
            val = (mx.e4m3_value if fmt == "e4m3" else mx.e2m1_value)(codes[r, 32 * b + big])
            assert 2.0 ** emax <= abs(val) <= (448.0 if fmt == "e4m3" else 6.0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_power_of_two_scaling(fmt):
    g = np.random.default_rng(3)
    x = (g.standard_normal((4, 96)) * 3).astype(np.float16)
    c0, s0 = mx.mx_quantize(x, fmt)
    for k in (-5, -1, 2, 6):
        c1, s1 = mx.mx_quantize((x.astype(np.float64) * 2.0 ** k).astype(np.float16), fmt)
        assert np.array_equal(c1, c0)
        assert np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_zero_block():
    x = np.zeros((2, 64), np.float16)
    x[1, 40] = 1.0
    for fmt in ("e4m3", "e2m1"):
        c, s = mx.mx_quantize(x, fmt)
        assert c[0].tolist() == [0] * 64 and s[0].tolist() == [0, 0]
        assert s[1, 0] == 0 and c[1, :32].tolist() == [0] * 32


def _representable_block(g, table_vals, top):
    """32 values from a format's grid whose largest magnitude is `top` (scale code 127)."""
    v = g.choice(table_vals, size=32) * g.choice([-1.0, 1.0], size=32)
    v[g.integers(32)] = top * g.choice([-1.0, 1.0])
    return v


def test_lossless_product_is_plain_matmul():
    """Inputs already on the MX grids with block maxima in the top binade: conversion is
    lossless, so the product equals np.matmul of the raw inputs."""
    g = np.random.default_rng(4)
    e4m3_grid = mx.e4m3_value(np.arange(0x7F))
    m, n, k = 5, 7, 128
    x = np.concatenate([np.stack([_representable_block(g, e4m3_grid, 448.0 if r % 2 else 320.0)
                                  for _ in range(k // 32)]).reshape(-1) for r in range(m)]).reshape(m, k)
    w = np.concatenate([np.stack([_representable_block(g, np.array(E2M1_TABLE), 6.0 if r % 2 else 4.0)
                                  for _ in range(k // 32)]).reshape(-1) for r in range(n)]).reshape(n, k)
    x16, w16 = x.astype(np.float16), w.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x) and np.array_equal(w16.astype(np.float64), w)
    _, sa = mx.mx_quantize(x16, "e4m3")
    _, sw = mx.mx_quantize(w16, "e2m1")
    assert np.all(sa == 127) and np.all(sw == 127)
    assert np.array_equal(mx.mx_linear(x16, w16), x @ w.T)


def test_product_scales_exactly():
    g = np.random.default_rng(5)
    x = (g.standard_normal((3, 64)) * 2).astype(np.float16)
    w = (g.standard_normal((4, 64)) * 0.05).astype(np.float16)
    base = mx.mx_linear(x, w)
    x2 = (x.astype(np.float64) * 8).astype(np.float16)
    w2 = (w.astype(np.float64) / 4).astype(np.float16)
    assert np.array_equal(mx.mx_linear(x2, w2), base * 2)


def test_abs_terms_equals_product_for_nonnegative_inputs():
    """sum |a w| (the tolerance helper) is the product itself when every term is nonnegative."""
    g = np.random.default_rng(6)
    x = np.abs(g.standard_normal((3, 96))).astype(np.float16)
    w = np.abs(g.standard_normal((5, 96)) * 0.1).astype(np.float16)
    qa, sa = mx.mx_quantize(x, "e4m3")
    qw, sw = mx.mx_quantize(w, "e2m1")
    assert np.allclose(mx.mx_abs_terms(qa, sa, qw, sw), mx.mx_linear(x, w), rtol=1e-15, atol=0)
