"""GPU parity of the small-batch kernel (W4A8_PATH_BATCH: 1 .. 16 token rows on the int8
matrix instruction) against the CPU oracle.

Integer block sums must match bit for bit; fp32 outputs must satisfy
|gpu - ref| <= 1e-3 + 1e-3 * |ref| against the oracle's fp64 result.  The shapes
cover one and several rounds of weight loads per wave, a last round with fewer
blocks than the others, both row tilings (up to 8 rows, up to 16) and the
wide workload (K = 4096, N = 14336) at full size.
"""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL = 1e-3
RTOL = 1e-3
BATCH = w4.PATH_BATCH


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    bad = int((excess > 0).sum())
    assert bad == 0, f"{what}: {bad} of {ref.size} outside tolerance, max excess {excess.max():.3g}"


# K = 256 is one block per wave; 768 three (a round of 8 with 3 valid); 2048 eight; 4096
# sixteen (one round of 16); 5120 twenty (a round of 16, then one with 4 valid).
SHAPES = [(1, 256, 64), (2, 768, 192), (3, 2048, 128), (5, 5120, 64), (8, 4096, 320), (9, 256, 64),
          (12, 768, 192), (13, 5120, 128), (16, 4096, 1024), (16, 2048, 64)]


@pytest.mark.parametrize("m,k,n", SHAPES)
def test_block_sums_bit_exact(m, k, n):
    x, qw, sw = synth.linear_inputs(m * 31 + k + n, m, k, n, outliers=True)
    packed, _ = w4.pack_weights(dev(qw), dev(sw))
    got = host(w4.block_sums(dev(x), packed, path=BATCH))
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw)), f"M={m} K={k} N={n}"


@pytest.mark.parametrize("m,k,n", SHAPES)
def test_linear_against_oracle(m, k, n):
    x, qw, sw = synth.linear_inputs(m * 17 + k + n, m, k, n, outliers=True)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    got = host(w4.linear(dev(x), packed, ws, path=BATCH))
    assert_close(got, oracle.linear(x, qw, sw), f"M={m} K={k} N={n}")


@pytest.mark.parametrize("m", list(range(1, 17)))
def test_every_row_count(m):
    """Rows past M are zero codes in the matrix operand: every M from 1 to 16 at a shape with
    two rounds of weight loads."""
    k, n = 5120, 192
    x, qw, sw = synth.linear_inputs(900 + m, m, k, n, outliers=True)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    xd = dev(x)
    assert_close(host(w4.linear(xd, packed, ws, path=BATCH)), oracle.linear(x, qw, sw), f"M={m}")
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(host(w4.block_sums(xd, packed, path=BATCH)).astype(np.int64), oracle.block_sums(qx, qw))


def test_block_sums_extreme_values():
    """All codes at their extremes: |I| reaches 32 * 127 * 8 = 32512 in every block and row."""
    m, k, n = 16, 512, 64
    x = np.full((m, k), 3.0, dtype=np.float16)
    x[1::2] = -3.0
    qw = np.full((n, k), -8, dtype=np.int8)
    qw[1::2] = 7
    sw = np.ones((n, k // 32), dtype=np.float16)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    got = host(w4.block_sums(dev(x), packed, path=BATCH))
    assert got[0, 0, 0] == -32512 and got[1, 0, 0] == 32512
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))
    assert_close(host(w4.linear(dev(x), packed, ws, path=BATCH)), oracle.linear(x, qw, sw), "extremes")


def test_special_values_bit_exact():
    """Codes decided by the kernel's own quantiser: fp16 subnormals, exact ties of x / sx (every
    element takes the exact-division fallback), the fp16 maximum and negative zeros."""
    g = np.random.default_rng(5)
    x = np.zeros((4, 256), dtype=np.float16)
    x[1] = (g.integers(-1023, 1024, 256) * 2.0 ** -24).astype(np.float16)
    x[2] = (g.integers(-254, 255, 256) / 2.0).astype(np.float16)
    x[2, ::32] = 127.0
    x[3] = np.clip(g.standard_normal(256) * 2e4, -65504, 65504).astype(np.float16)
    x[3, 7] = 65504.0
    x[3, 64:96] = -0.0
    _, qw, sw = synth.linear_inputs(8, 4, 256, 64)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    qx, _ = oracle.quantize_activations(x)
    got = host(w4.block_sums(dev(x), packed, path=BATCH))
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))
    assert_close(host(w4.linear(dev(x), packed, ws, path=BATCH)), oracle.linear(x, qw, sw), "special values")


def test_zero_and_outlier_rows():
    """All-zero rows give exact zeros; rows scaled to the fp16 range stay within tolerance."""
    m, k, n = 16, 2048, 256
    x, qw, sw = synth.linear_inputs(77, m, k, n, outliers=True)
    x[3] = 0.0
    x[11] = 0.0
    x[5] = (x[5].astype(np.float32) * 1000.0).clip(-65504, 65504).astype(np.float16)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    got = host(w4.linear(dev(x), packed, ws, path=BATCH))
    assert np.all(got[3] == 0.0) and np.all(got[11] == 0.0)
    assert_close(got, oracle.linear(x, qw, sw), "zero and outlier rows")


@pytest.mark.parametrize("m", [m for m in synth.WORKLOADS["wide"]["M"] if m <= 16])
def test_wide_workload_full(m):
    x, qw, sw = synth.workload_inputs("wide", m)["wide"]
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    got = host(w4.linear(dev(x), packed, ws, path=BATCH))
    assert_close(got, oracle.linear(x, qw, sw), f"wide M={m}")


def test_repeat_runs_are_bit_identical():
    x, qw, sw = synth.linear_inputs(5, 11, 4096, 1024, outliers=True)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    xd = dev(x)
    a = host(w4.linear(xd, packed, ws, path=BATCH))
    b = host(w4.linear(xd, packed, ws, path=BATCH))
    assert np.array_equal(a.view(np.int32), b.view(np.int32))


def test_every_step_waits_for_both_quantiser_waves():
    """Repeated calls at shapes whose MFMAs start as soon as a step's activations are in
    LDS: every call must match the oracle (a step may not start on one quantiser wave's
    half of the rows)."""
    for m, k, n in [(16, 2048, 128), (16, 1024, 64), (11, 2048, 192)]:
        x, qw, sw = synth.linear_inputs(m + k + n, m, k, n, outliers=True)
        packed, ws = w4.pack_weights(dev(qw), dev(sw))
        xd = dev(x)
        qx, _ = oracle.quantize_activations(x)
        ref = oracle.block_sums(qx, qw)
        for rep in range(20):
            got = host(w4.block_sums(xd, packed, path=BATCH)).astype(np.int64)
            assert np.array_equal(got, ref), f"M={m} K={k} N={n} call {rep}"


def test_graph_replay_matches_eager_calls():
    """Captured in a HIP graph (the kernel uses no scratch and no memset), replays with new
    activations written in place between them match eager calls bit for bit."""
    m, k, n = 12, 4096, 1024
    _, qw, sw = synth.linear_inputs(31, m, k, n, outliers=True)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    xs = [synth.linear_inputs(40 + i, m, k, n, outliers=True)[0] for i in range(3)]
    xd = dev(xs[0])
    out = torch.empty((m, n), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w4.linear(xd, packed, ws, path=BATCH, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.linear(xd, packed, ws, path=BATCH, out=out)
    for i, x in enumerate(xs + xs[:1]):
        xd.copy_(dev(x))
        g.replay()
        got = host(out).copy()
        ref = host(w4.linear(dev(x), packed, ws, path=BATCH))
        assert np.array_equal(got.view(np.int32), ref.view(np.int32)), f"replay {i}"


def test_rejected_shapes_raise():
    x, qw, sw = synth.linear_inputs(6, 17, 256, 64)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    with pytest.raises(w4.W4A8Error):
        w4.linear(dev(x), packed, ws, path=BATCH)
    x, qw, sw = synth.linear_inputs(6, 2, 288, 64)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    with pytest.raises(w4.W4A8Error):
        w4.linear(dev(x), packed, ws, path=BATCH)
