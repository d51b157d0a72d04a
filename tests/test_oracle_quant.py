"""Pins of the oracle's activation quantiser (not the GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _golden_blocks():
    with open(os.path.join(GOLDEN, "quant_blocks.json")) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b["name"])
def test_golden_block(blk):
    x = np.array([blk["x"]], dtype=np.float16)
    q, sx = oracle.quantize_activations(x)
    assert sx.dtype == np.float32 and q.dtype == np.int8
    assert sx[0, 0] == np.float32(blk["sx"])
    assert q[0].tolist() == blk["q"]


def test_golden_blocks_side_by_side():
    """All golden blocks in one row: each block is quantised on its own."""
    blocks = _golden_blocks()
    x = np.array([sum((b["x"] for b in blocks), [])], dtype=np.float16)
    q, sx = oracle.quantize_activations(x)
    assert sx[0].tolist() == [b["sx"] for b in blocks]
    assert q[0].tolist() == sum((b["q"] for b in blocks), [])


def _random_x(seed, m=16, k=256, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "normal":
        x = g.standard_normal((m, k))
    elif kind == "outliers":
        x = g.standard_normal((m, k))
        x[:, g.choice(k, 5, replace=False)] *= 20
    elif kind == "wide":
        x = g.standard_normal((m, k)) * np.exp2(g.integers(-12, 12, size=(m, k)))
    elif kind == "ties":
        x = (g.integers(-254, 255, size=(m, k)) / 2.0)
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


@pytest.mark.parametrize("kind", ["normal", "outliers", "wide", "ties"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rounding_error_bound(kind, seed):
    """|x/sx - q| <= 1/2 + 127 * 2**-24 (half a step plus the fp32 rounding of x/sx), |q| <= 127."""
    x = _random_x(seed, kind=kind)
    q, sx = oracle.quantize_activations(x)
    m, k = x.shape
    xb = x.astype(np.float64).reshape(m, k // 32, 32)
    qb = q.astype(np.float64).reshape(m, k // 32, 32)
    s = sx.astype(np.float64)[:, :, None]
    assert np.abs(q).max() <= 127
    nz = s[:, :, 0] > 0
    err = np.abs(xb / np.where(s > 0, s, 1.0) - qb)
    assert np.all(err[nz] <= 0.5 + 127 * 2.0 ** -24)
    assert np.all(qb[~nz] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_amax_element_reaches_full_scale(seed):
    x = _random_x(seed, kind="wide")
    q, sx = oracle.quantize_activations(x)
    m, k = x.shape
    xb = x.astype(np.float32).reshape(m, k // 32, 32)
    qb = q.reshape(m, k // 32, 32)
    idx = np.argmax(np.abs(xb), axis=2)
    top_q = np.take_along_axis(qb, idx[:, :, None], axis=2)[:, :, 0]
    top_x = np.take_along_axis(xb, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top_q.astype(int)) == 127)
    assert np.all(np.sign(top_q) == np.sign(top_x))
    # sx is the fp32 quotient amax / 127
    assert np.all(sx == (np.abs(top_x) / np.float32(127)).astype(np.float32))


@pytest.mark.parametrize("j", [-4, -1, 1, 3])
def test_power_of_two_invariance(j):
    """Scaling x by 2**j (exact in fp16 here) leaves q unchanged and scales sx exactly."""
    g = np.random.default_rng(7)
    mag = np.exp2(g.uniform(-8, 3, size=(8, 128)))
    x = (mag * g.choice([-1.0, 1.0], size=mag.shape)).astype(np.float16)
    xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
    assert np.all(xs.astype(np.float64) == x.astype(np.float64) * 2.0 ** j)
    q0, s0 = oracle.quantize_activations(x)
    q1, s1 = oracle.quantize_activations(xs)
    assert np.array_equal(q0, q1)
    assert np.all(s1.astype(np.float64) == s0.astype(np.float64) * 2.0 ** j)


def test_sign_symmetry():
    x = _random_x(5, kind="ties")
    q0, s0 = oracle.quantize_activations(x)
    q1, s1 = oracle.quantize_activations(-x)
    assert np.array_equal(q1, -q0) and np.array_equal(s0, s1)


def test_fp16_subnormal_blocks():
    """Blocks of fp16 subnormals quantise like the same integers scaled by 2**-24."""
    g = np.random.default_rng(3)
    ints = g.integers(-1023, 1024, size=(4, 64)).astype(np.float64)
    ints[:, 0] = 1000.0                       # keep every block non-zero
    ints[:, 32] = -1000.0
    x_int = ints.astype(np.float16)
    x_sub = (ints * 2.0 ** -24).astype(np.float16)
    assert np.all(np.abs(x_sub[x_sub != 0]).astype(np.float64) < 2.0 ** -14)   # all subnormal
    assert np.all(x_sub.astype(np.float64) == ints * 2.0 ** -24)
    q0, s0 = oracle.quantize_activations(x_int)
    q1, s1 = oracle.quantize_activations(x_sub)
    assert np.array_equal(q0, q1)
    assert np.all(s1.astype(np.float64) == s0.astype(np.float64) * 2.0 ** -24)


def test_zero_block_inside_row():
    x = _random_x(9, m=2, k=96)
    x[:, 32:64] = 0
    q, sx = oracle.quantize_activations(x)
    assert np.all(sx[:, 1] == 0) and np.all(q[:, 32:64] == 0)
    assert np.all(sx[:, [0, 2]] > 0)


def test_rejects_non_finite():
    x = np.zeros((1, 32), dtype=np.float16)
    x[0, 3] = np.inf
    with pytest.raises(AssertionError):
        oracle.quantize_activations(x)


def _division_blocks():
    with open(os.path.join(GOLDEN, "quant_division_blocks.json")) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _division_blocks(), ids=lambda b: b["name"])
def test_division_block(blk):
    """Non-power-of-two scales: codes derived with exact rational arithmetic
    (tests/golden/make_quant_division_blocks.py), where a reciprocal multiply
    or a reciprocal scale would round some elements the other way."""
    x = np.array([blk["x"]], dtype=np.float16)
    assert x.astype(np.float64)[0].tolist() == blk["x"]
    q, sx = oracle.quantize_activations(x)
    assert sx[0, 0] == np.float32(blk["sx"])
    assert q[0].tolist() == blk["q"]


def test_division_blocks_tell_the_shortcuts_apart():
    """The fixture only pins the division if the shortcuts give other codes somewhere."""
    blocks = _division_blocks()
    assert any(b["q"] != b["q_if_reciprocal_multiply"] for b in blocks)
    assert any(b["q"] != b["q_if_inverse_scale"] for b in blocks)
    assert any(b["q"] != b["q_if_scale_times_rcp127"] or b["sx"] != b["sx_if_scale_times_rcp127"]
               for b in blocks)
    for b in blocks:
        s = np.float32(b["sx"])
        m, _ = np.frexp(s)
        assert m != 0.5, "scale must not be a power of two"
