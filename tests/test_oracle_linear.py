"""Pins of the oracle's block sums, scaled output and argmax (not the GPU)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def test_golden_linear():
    with open(os.path.join(GOLDEN, "linear_examples.json")) as f:
        d = json.load(f)
    x = np.array(d["x"], dtype=np.float16)
    qw = np.array(d["qw"], dtype=np.int8)
    sw = np.array(d["sw"], dtype=np.float16)
    qx, sx = oracle.quantize_activations(x)
    assert oracle.block_sums(qx, qw).tolist() == d["block_sums"]
    assert oracle.linear(x, qw, sw).tolist() == d["out"]


def _tiny(seed, m, k, n):
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float16)
    qw = g.integers(-8, 8, size=(n, k)).astype(np.int8)
    sw = g.uniform(0.005, 0.02, size=(n, k // 32)).astype(np.float16)
    return x, qw, sw


@pytest.mark.parametrize("seed,m,k,n", [(0, 2, 64, 3), (1, 1, 32, 5), (2, 3, 96, 2)])
def test_block_sums_brute_force(seed, m, k, n):
    x, qw, _ = _tiny(seed, m, k, n)
    qx, _ = oracle.quantize_activations(x)
    got = oracle.block_sums(qx, qw)
    for mm, nn, b in itertools.product(range(m), range(n), range(k // 32)):
        want = 0
        for j in range(32):
            want += int(qx[mm, 32 * b + j]) * int(qw[nn, 32 * b + j])
        assert got[mm, nn, b] == want


def test_extreme_block_sums_are_exact():
    qx = np.full((2, 64), 127, dtype=np.int8)
    qx[1] = -127
    qw = np.full((3, 64), -8, dtype=np.int8)
    got = oracle.block_sums(qx, qw)
    assert np.all(got[0] == -32512) and np.all(got[1] == 32512)


def test_integer_gemm_special_case():
    """K = 32, unit weight scales, integer x with max|x| = 127 per row: out == qx @ qw.T exactly."""
    g = np.random.default_rng(4)
    m, n = 7, 9
    xi = g.integers(-127, 128, size=(m, 32))
    xi[:, 5] = 127
    x = xi.astype(np.float16)
    qw = g.integers(-8, 8, size=(n, 32)).astype(np.int8)
    sw = np.ones((n, 1), dtype=np.float16)
    out = oracle.linear(x, qw, sw)
    want = xi.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(out, want.astype(np.float64))


@pytest.mark.parametrize("seed,m,k,n", [(0, 3, 96, 5), (1, 4, 64, 7), (5, 1, 256, 3)])
def test_dequantize_then_matmul(seed, m, k, n):
    """Scaling each block then summing equals dequantising both operands and one fp64 matmul."""
    x, qw, sw = _tiny(seed, m, k, n)
    qx, sx = oracle.quantize_activations(x)
    xh = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 32, axis=1)
    wh = qw.astype(np.float64) * np.repeat(sw.astype(np.float64), 32, axis=1)
    want = xh @ wh.T
    got = oracle.linear(x, qw, sw)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_power_of_two_scale_invariants():
    x, qw, sw = _tiny(8, 3, 128, 6)
    base = oracle.linear(x, qw, sw)
    sw2 = (sw.astype(np.float64) * 2).astype(np.float16)
    assert np.array_equal(oracle.linear(x, qw, sw2), 2 * base)
    x4 = (x.astype(np.float64) * 4).astype(np.float16)
    assert np.array_equal(oracle.linear(x4, qw, sw), 4 * base)


def test_column_subset_consistency():
    x, qw, sw = _tiny(12, 2, 64, 10)
    full = oracle.linear(x, qw, sw)
    cols = [7, 2, 9]
    assert np.array_equal(oracle.linear(x, qw[cols], sw[cols]), full[:, cols])


def _scan_argmax(row):
    best = 0
    for i in range(1, len(row)):
        if row[i] > row[best]:
            best = i
    return best


def test_argmax_against_scan():
    g = np.random.default_rng(2)
    v = g.standard_normal((6, 1000)).astype(np.float32)
    v[1, 10] = v[1, 700] = 50.0          # tie: lowest index wins
    v[2, :] = 0.0
    v[2, 300] = -0.0                      # all zeros with a signed zero: index 0
    v[3, :] = -1.0
    v[3, 5] = -0.0
    v[3, 4] = 0.0                         # +0 at 4 and -0 at 5 tie: 4
    v[4, 999] = 1e30
    got = oracle.argmax_first(v)
    assert got.tolist() == [_scan_argmax(r) for r in v]
    assert got[1] == 10 and got[2] == 0 and got[3] == 4 and got[4] == 999
