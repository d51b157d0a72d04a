"""Pins of the oracle's decoder-layer glue (not the GPU)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_rms_norm_constant_rows():
    """A constant row c normalises to fp16(c / sqrt(c^2 + eps)): +-1 for eps = 0."""
    x = np.array([[3.0] * 64, [-0.25] * 64, [1e-3] * 64], dtype=np.float32)
    y = oracle.rms_norm_fp16(x, 0.0)
    assert np.all(y[0] == 1.0) and np.all(y[1] == -1.0) and np.all(y[2] == 1.0)
    y = oracle.rms_norm_fp16(np.full((1, 8), 2.0, np.float32), 12.0)   # 2 / sqrt(4 + 12) = 0.5
    assert np.all(y == 0.5)


def test_rms_norm_power_of_two_invariance_and_unit_mean_square():
    g = np.random.default_rng(0)
    x = g.standard_normal((4, 256)).astype(np.float32)
    y0 = oracle.rms_norm_fp16(x, 0.0)
    for j in (-5, 3, 9):
        assert np.array_equal(oracle.rms_norm_fp16((x * 2.0 ** j).astype(np.float32), 0.0), y0)
    ms = np.mean(y0.astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) < 2e-3)


def test_residual_add_is_one_rounding():
    g = np.random.default_rng(1)
    x = (g.standard_normal(200) * 10).astype(np.float32)
    d = (g.standard_normal(200) * 1000).astype(np.float32)
    got = oracle.residual_add(x[None], d[None], 0.01)[0]
    a = Fraction(float(np.float32(0.01)))
    for xi, di, gi in zip(x, d, got):
        exact = Fraction(float(xi)) + a * Fraction(float(di))
        lo = np.float32(float(exact))
        # the float32 nearest to the exact value: compare both neighbours
        cands = [lo, np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(-np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact), int(np.frombuffer(c.tobytes(), np.uint32)[0]) & 1))
        assert gi == best


def test_gated_product_hand_example():
    g = np.array([[2.0, 3.0, 0.5, -4.0]], dtype=np.float32)   # F = 2: [2*0.5, 3*-4]
    assert oracle.gated_fp16(g).tolist() == [[1.0, -12.0]]
    big = np.array([[300.0, 1.0, 300.0, 1.0]], dtype=np.float32)   # 90000 overflows fp16
    with np.errstate(over="ignore"):
        assert np.isinf(oracle.gated_fp16(big)[0, 0])


def _layer_weights(seed, h=64, n_qkv=128, f=128, zero=()):
    g = np.random.default_rng(seed)
    shapes = {"qkv": (h, n_qkv), "o": (h, h), "gate_up": (h, 2 * f), "down": (f, h)}
    w = {}
    for name, (k, n) in shapes.items():
        qw = g.integers(-8, 8, size=(n, k)).astype(np.int8)
        if name in zero:
            qw[:] = 0
        sw = g.uniform(0.005, 0.02, size=(n, k // 32)).astype(np.float16)
        w[name] = (qw, sw)
    return w


def test_layer_with_zero_weights_is_identity():
    x = np.random.default_rng(2).standard_normal((3, 64)).astype(np.float32)
    w = _layer_weights(3, zero=("qkv", "o", "gate_up", "down"))
    assert np.array_equal(oracle.decoder_layer(x, w, 0.01, 1e-6), x)


def test_layer_without_feed_forward_adds_only_the_attention_path():
    x = np.random.default_rng(4).standard_normal((2, 64)).astype(np.float32)
    w = _layer_weights(5, zero=("down",))
    got = oracle.decoder_layer(x, w, 0.01, 1e-6)
    n1 = oracle.rms_norm_fp16(x, 1e-6)
    q = oracle.linear_fp32(n1, *w["qkv"])
    o = oracle.linear_fp32(q[:, :64].astype(np.float16), *w["o"])
    assert np.array_equal(got, oracle.residual_add(x, o, 0.01))
    assert not np.array_equal(got, x)


@pytest.mark.parametrize("seed", [0, 1])
def test_layer_keeps_the_residual_stream_bounded(seed):
    """With the 0.01 residual scale and normalised layer inputs the stream changes by a few percent."""
    x = np.random.default_rng(seed).standard_normal((2, 64)).astype(np.float32)
    w = _layer_weights(10 + seed)
    y = oracle.decoder_layer(x, w, 0.01, 1e-6)
    rel = np.linalg.norm(y - x) / np.linalg.norm(x)
    assert 1e-4 < rel < 0.5


def _zeroed(w, name, rows=None):
    """A copy of w with the weights of `name` zeroed (all rows, or rows[0]:rows[1])."""
    out = {k: (v[0].copy(), v[1]) for k, v in w.items()}
    qw = out[name][0]
    if rows is None:
        qw[:] = 0
    else:
        qw[rows[0]:rows[1]] = 0
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_feed_forward_reads_the_stream_after_attention(seed):
    """The feed-forward half normalises x after the attention residual add.

    layer(x) equals two layer calls: the first without the feed-forward path
    (down = 0, so it returns x after attention exactly), the second without
    the attention path (o = 0, so its attention add is exact and its
    feed-forward path sees the first call's result).  A layer whose
    feed-forward path normalised the pre-attention x, or added d to it, would
    differ."""
    x = np.random.default_rng(20 + seed).standard_normal((3, 64)).astype(np.float32)
    w = _layer_weights(30 + seed)
    whole = oracle.decoder_layer(x, w, 0.01, 1e-6)
    after_attention = oracle.decoder_layer(x, _zeroed(w, "down"), 0.01, 1e-6)
    assert not np.array_equal(after_attention, x)
    two_calls = oracle.decoder_layer(after_attention, _zeroed(w, "o"), 0.01, 1e-6)
    assert np.array_equal(whole, two_calls)
    # and the feed-forward path of the second call does change the stream
    assert not np.array_equal(two_calls, after_attention)


@pytest.mark.parametrize("half", ["gate", "up"])
def test_feed_forward_needs_both_halves_of_gate_up(half):
    """u = fp16(gate * up): with either half of gate/up zero the product is
    zero and the feed-forward path adds nothing (the same result as down = 0)."""
    x = np.random.default_rng(40).standard_normal((2, 64)).astype(np.float32)
    f = 128
    w = _layer_weights(41, f=f)
    rows = (0, f) if half == "gate" else (f, 2 * f)
    got = oracle.decoder_layer(x, _zeroed(w, "gate_up", rows), 0.01, 1e-6)
    assert np.array_equal(got, oracle.decoder_layer(x, _zeroed(w, "down"), 0.01, 1e-6))
    assert not np.array_equal(oracle.decoder_layer(x, w, 0.01, 1e-6), got)


def test_attention_path_reads_only_the_query_slice():
    """a = fp16(q[:, :H]): qkv columns past H never matter, and with the first H
    zero the attention path adds nothing (the same result as o = 0)."""
    x = np.random.default_rng(50).standard_normal((2, 64)).astype(np.float32)
    w = _layer_weights(51, n_qkv=192)
    whole = oracle.decoder_layer(x, w, 0.01, 1e-6)
    assert np.array_equal(oracle.decoder_layer(x, _zeroed(w, "qkv", (64, 192)), 0.01, 1e-6), whole)
    no_query = oracle.decoder_layer(x, _zeroed(w, "qkv", (0, 64)), 0.01, 1e-6)
    assert np.array_equal(no_query, oracle.decoder_layer(x, _zeroed(w, "o"), 0.01, 1e-6))
    assert not np.array_equal(no_query, whole)
