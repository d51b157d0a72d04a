"""The seeded generators: shapes, ranges and reproducibility (no method arithmetic here)."""
import numpy as np

import synth


def test_linear_inputs_shapes_and_ranges():
    x, qw, sw = synth.linear_inputs(0, 3, 2048, 128, outliers=True)
    assert x.dtype == np.float16 and x.shape == (3, 2048)
    assert qw.dtype == np.int8 and qw.shape == (128, 2048)
    assert qw.min() == -8 and qw.max() == 7
    assert sw.dtype == np.float16 and sw.shape == (128, 64)
    assert sw.min() >= np.float16(0.005) and sw.max() <= np.float16(0.02)


def test_reproducible():
    a = synth.linear_inputs(3, 2, 256, 64)
    b = synth.linear_inputs(3, 2, 256, 64)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    c = synth.linear_inputs(4, 2, 256, 64)
    assert not np.array_equal(a[1], c[1])


def test_outlier_channel_counts():
    for k, want in [(2048, 20), (4096, 41), (8192, 82)]:
        ch = synth.outlier_channels(synth.rng(0, 0), k)
        assert len(ch) == want and len(set(ch.tolist())) == want
        assert ch.min() >= 0 and ch.max() < k


def test_outlier_channels_are_amplified():
    g = synth.rng(1, 3)
    ch = synth.outlier_channels(g, 2048)
    x = synth.activations(synth.rng(1, 2), 64, 2048, ch)
    mask = np.zeros(2048, bool)
    mask[ch] = True
    ratio = np.abs(x[:, mask].astype(float)).mean() / np.abs(x[:, ~mask].astype(float)).mean()
    assert 15 < ratio < 25


def test_workload_tables():
    w = synth.workload_inputs("single")
    x, qw, sw = w["single"]
    assert x.shape == (1, 2048) and qw.shape == (2048, 2048)
    assert synth.LAYER_SHAPES["down"] == (8192, 2048)
