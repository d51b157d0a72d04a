"""Pins of the oracle's int4 packer (not the GPU)."""
import json
import os

import numpy as np

import oracle
from conftest import GOLDEN


def test_golden_layout():
    with open(os.path.join(GOLDEN, "pack_layout.json")) as f:
        d = json.load(f)
    qw = np.array(d["qw"], dtype=np.int8)
    sw = np.array(d["sw"], dtype=np.float16)
    packed, ws = oracle.pack_weights(qw, sw)
    assert packed.shape == (d["K"] // 32, d["N"], 16)
    flat = [bytes(packed[b, n]).hex() for b in range(packed.shape[0]) for n in range(packed.shape[1])]
    assert flat == d["packed_hex"]
    assert ws.astype(np.float64).tolist() == d["w_scales"]
    q2, s2 = oracle.unpack_weights(packed, ws)
    assert np.array_equal(q2, qw) and np.array_equal(s2, sw)


def test_every_nibble_in_every_position():
    """Column c holds value ((c + j) % 16) - 8 at position j: all 16 values at all 32 positions."""
    n, k = 16, 64
    c = np.arange(n)[:, None]
    j = np.arange(k)[None, :]
    qw = (((c + j) % 16) - 8).astype(np.int8)
    sw = np.ones((n, k // 32), dtype=np.float16)
    packed, ws = oracle.pack_weights(qw, sw)
    q2, _ = oracle.unpack_weights(packed, ws)
    assert np.array_equal(q2, qw)
    # byte j of block b holds elements 32b+j (low) and 32b+16+j (high)
    for b in range(k // 32):
        for jj in range(16):
            byte = packed[b, :, jj].astype(int)
            lo = np.where((byte & 0xF) >= 8, (byte & 0xF) - 16, byte & 0xF)
            hi = np.where((byte >> 4) >= 8, (byte >> 4) - 16, byte >> 4)
            assert np.array_equal(lo, qw[:, 32 * b + jj])
            assert np.array_equal(hi, qw[:, 32 * b + 16 + jj])


def test_random_round_trip():
    g = np.random.default_rng(11)
    qw = g.integers(-8, 8, size=(192, 256)).astype(np.int8)
    sw = g.uniform(0.005, 0.02, size=(192, 8)).astype(np.float16)
    packed, ws = oracle.pack_weights(qw, sw)
    assert packed.dtype == np.uint8 and ws.dtype == np.float16
    assert ws.shape == (8, 192)
    q2, s2 = oracle.unpack_weights(packed, ws)
    assert np.array_equal(q2, qw) and np.array_equal(s2, sw)
