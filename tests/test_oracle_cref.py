"""The plain C reference (oracle/w4a8_ref.c) against the pinned numpy oracle, bit for bit."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN
from oracle import cref


def _blocks(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("name", ["quant_blocks.json", "quant_division_blocks.json"])
def test_golden_blocks(name):
    for blk in _blocks(name):
        q, sx = cref.quantize(np.array([blk["x"]], dtype=np.float16))
        assert sx[0, 0] == np.float32(blk["sx"]), blk["name"]
        assert q[0].tolist() == blk["q"], blk["name"]


def _inputs(kind, seed, m=9, k=320):
    g = np.random.default_rng(seed)
    if kind == "normal":
        x = g.standard_normal((m, k))
    elif kind == "outliers":
        x = g.standard_normal((m, k))
        x[:, g.choice(k, 7, replace=False)] *= 20
    elif kind == "wide":
        x = g.standard_normal((m, k)) * np.exp2(g.integers(-20, 14, size=(m, k)))
    elif kind == "subnormal":
        x = g.integers(-1023, 1024, size=(m, k)) * 2.0 ** -24
    elif kind == "ties":
        x = g.integers(-254, 255, size=(m, k)) / 2.0
    x = x.astype(np.float16)
    x[0, 32:64] = 0       # an all-zero block
    x[1, 64:96] = -0.0
    return x


@pytest.mark.parametrize("kind", ["normal", "outliers", "wide", "subnormal", "ties"])
def test_quantize_equals_numpy_oracle(kind):
    x = _inputs(kind, 3)
    q0, s0 = oracle.quantize_activations(x)
    q1, s1 = cref.quantize(x)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_block_sums_equal_numpy_oracle():
    x, qw, _ = synth.linear_inputs(11, 5, 256, 192, outliers=True)
    qx, _ = oracle.quantize_activations(x)
    ref = oracle.block_sums(qx, qw)
    assert np.array_equal(cref.block_sums(qx, qw, threads=1), ref)
    assert np.array_equal(cref.block_sums(qx, qw, threads=4), ref)


@pytest.mark.parametrize("m,k,n,outliers", [(1, 2048, 256, False), (7, 512, 320, True), (3, 96, 64, True)])
def test_linear_equals_numpy_oracle(m, k, n, outliers):
    """Identical fp64 outputs: both sum I * sw * sx over blocks in ascending order."""
    x, qw, sw = synth.linear_inputs(m + k + n, m, k, n, outliers=outliers)
    ref = oracle.linear(x, qw, sw)
    got1 = cref.linear(x, qw, sw, threads=1)
    got8 = cref.linear(x, qw, sw, threads=8)
    assert np.array_equal(got1, ref)
    assert np.array_equal(got8, ref)


def test_golden_linear_example():
    with open(os.path.join(GOLDEN, "linear_examples.json")) as f:
        d = json.load(f)
    x = np.array(d["x"], dtype=np.float16)
    qw = np.array(d["qw"], dtype=np.int8)
    sw = np.array(d["sw"], dtype=np.float16)
    qx, _ = cref.quantize(x)
    assert cref.block_sums(qx, qw).tolist() == d["block_sums"]
    assert cref.linear(x, qw, sw).tolist() == d["out"]
