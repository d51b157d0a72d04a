"""Pins of the decode-attention oracle (oracle/attention.py) against closed forms and
invariants of softmax attention: one position, two positions through the logistic
function (which fixes the 1/sqrt(D) scale and the sign), uniform weights giving the
mean, the grouped-query head mapping, invariance to the order of positions and to a
common shift of all scores, a dominant key, stability at large scores, and a scalar
brute-force loop on a tiny case."""
import math

import numpy as np
import pytest

from oracle import attention as at
from synth import attention_inputs


def _empty(hkv, d):
    return np.zeros((hkv, 0, d), np.float16)


def test_single_position_returns_the_new_value():
    g = np.random.default_rng(0)
    q = g.standard_normal((4, 64)).astype(np.float32)
    k_new = g.standard_normal((2, 64)).astype(np.float32)
    v_new = g.standard_normal((2, 64)).astype(np.float32)
    out = at.decode_attention(q, k_new, v_new, _empty(2, 64), _empty(2, 64))
    v16 = v_new.astype(np.float16)
    assert np.array_equal(out, v16[[0, 0, 1, 1]])


def test_two_positions_follow_the_logistic_function():
    """q = 2 e_0, K_0 = 0, K_1 = 4 e_0, D = 64: s_1 - s_0 = 2 * 4 / 8 = 1, so
    out = V_0 + (V_1 - V_0) * sigma(1)."""
    d = 64
    q = np.zeros((1, d), np.float32)
    q[0, 0] = 2.0
    k_past = np.zeros((1, 1, d), np.float16)
    k_new = np.zeros((1, d), np.float32)
    k_new[0, 0] = 4.0
    g = np.random.default_rng(1)
    v_past = g.standard_normal((1, 1, d)).astype(np.float16)
    v_new = g.standard_normal((1, d)).astype(np.float16).astype(np.float32)
    out, _ = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    sigma = 1.0 / (1.0 + math.exp(-1.0))
    v0 = v_past[0, 0].astype(np.float64)
    v1 = v_new[0].astype(np.float64)
    assert np.allclose(out[0], v0 + (v1 - v0) * sigma, rtol=0, atol=1e-14)


def test_zero_query_gives_the_mean_value():
    q, k_new, v_new, k_past, v_past = attention_inputs(3, 4, 1, 128, 37)
    q[:] = 0.0
    out, _ = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    vals = np.concatenate([v_past[0].astype(np.float64), v_new.astype(np.float16).astype(np.float64)], axis=0)
    assert np.allclose(out, np.broadcast_to(vals.mean(axis=0), out.shape), rtol=0, atol=1e-14)


def test_grouped_query_heads_read_their_own_kv_head():
    """Hq = 6 over Hkv = 3: head h reads KV head h // 2; with V of KV head g constant g + 1
    the output of head h is exactly h // 2 + 1 (not h % 3 + 1)."""
    q, k_new, v_new, k_past, v_past = attention_inputs(4, 6, 3, 64, 20)
    for gi in range(3):
        v_past[gi] = gi + 1
        v_new[gi] = gi + 1
    out = at.decode_attention(q, k_new, v_new, k_past, v_past)
    assert np.array_equal(out, np.repeat(np.array([1, 1, 2, 2, 3, 3], np.float16)[:, None], 64, axis=1))


def test_order_of_past_positions_does_not_matter():
    q, k_new, v_new, k_past, v_past = attention_inputs(5, 8, 2, 64, 50)
    perm = np.random.default_rng(5).permutation(49)
    a, _ = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    b, _ = at.decode_attention_exact(q, k_new, v_new, k_past[:, perm], v_past[:, perm])
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_common_shift_of_every_key_cancels():
    """K_t + u for every t (the newest too) adds q.u / sqrt(D) to every score.  Keys and u
    sit on a grid of 1/4 so the shifted keys are exact in fp16."""
    g = np.random.default_rng(6)
    d, length = 64, 30
    q = g.standard_normal((2, d)).astype(np.float32)
    k_past = (g.integers(-12, 13, size=(1, length - 1, d)) / 4).astype(np.float16)
    k_new = (g.integers(-12, 13, size=(1, d)) / 4).astype(np.float32)
    u = g.integers(-8, 9, size=d) / 4
    v_past = g.standard_normal((1, length - 1, d)).astype(np.float16)
    v_new = g.standard_normal((1, d)).astype(np.float32)
    a, _ = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    b, _ = at.decode_attention_exact(q, (k_new + u).astype(np.float32), v_new,
                                     (k_past.astype(np.float64) + u).astype(np.float16), v_past)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value_at_large_scores():
    """A key aligned with q whose score exceeds the others by thousands: its value comes out
    (no overflow in the exponentials)."""
    q, k_new, v_new, k_past, v_past = attention_inputs(7, 2, 1, 64, 40)
    q[:] = 0.0
    q[:, 0] = 2000.0
    k_past[0, :, 0] = 0.0
    k_past[0, 17, 0] = 64.0          # score 2000 * 64 / 8 = 16000 vs 0 elsewhere
    k_new[0, 0] = 0.0
    out, _ = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    assert np.isfinite(out).all()
    assert np.array_equal(out, np.broadcast_to(v_past[0, 17].astype(np.float64), out.shape))


def test_probabilities_form_a_distribution():
    q, k_new, _, k_past, _ = attention_inputs(8, 8, 1, 256, 640)
    p = at.attention_probs(q, k_new, k_past)
    assert (p >= 0).all() and np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_new_key_and_value_enter_as_fp16():
    q, k_new, v_new, k_past, v_past = attention_inputs(9, 4, 1, 64, 10)
    a = at.decode_attention(q, k_new, v_new, k_past, v_past)
    b = at.decode_attention(q, k_new.astype(np.float16).astype(np.float32), v_new.astype(np.float16).astype(np.float32),
                            k_past, v_past)
    assert np.array_equal(a, b)


def test_scalar_brute_force_on_a_tiny_case():
    q, k_new, v_new, k_past, v_past = attention_inputs(10, 4, 2, 4, 3)
    out, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    for h in range(4):
        gi = h // 2
        keys = [[float(x) for x in k_past[gi, t]] for t in range(2)] + [[float(np.float16(x)) for x in k_new[gi]]]
        vals = [[float(x) for x in v_past[gi, t]] for t in range(2)] + [[float(np.float16(x)) for x in v_new[gi]]]
        scores = [sum(float(q[h, j]) * keys[t][j] for j in range(4)) / 2.0 for t in range(3)]
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        tot = sum(w)
        for j in range(4):
            assert out[h, j] == pytest.approx(sum(w[t] * vals[t][j] for t in range(3)) / tot, abs=1e-14)
            assert mag[h, j] == pytest.approx(sum(w[t] * abs(vals[t][j]) for t in range(3)) / tot, abs=1e-14)
