"""GPU parity: the HIP kernels behind the C ABI against the CPU oracle.

Integer and byte results (quantised activations, packed weights, integer block
sums, argmax indices) must match bit for bit; fp32 outputs must satisfy
|gpu - ref| <= 1e-3 + 1e-3 * |ref| against the oracle's fp64 result.
"""
import json
import os

import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth
from conftest import GOLDEN

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL = 1e-3
RTOL = 1e-3
PATHS = [w4.PATH_GEMV, w4.PATH_GEMM]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed_on_gpu(qw, sw):
    return w4.pack_weights(dev(qw), dev(sw))


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    bad = int((excess > 0).sum())
    assert bad == 0, f"{what}: {bad} of {ref.size} outside tolerance, max excess {excess.max():.3g}"


def inputs(seed, m, k, n, outliers=False):
    return synth.linear_inputs(seed, m, k, n, outliers=outliers)


# ----------------------------------------------------------------- quantiser
def test_quantize_golden_blocks():
    with open(os.path.join(GOLDEN, "quant_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    x = np.array([sum((b["x"] for b in blocks), [])], dtype=np.float16)
    qx, sx = w4.quantize_act(dev(x))
    assert host(sx)[0].tolist() == [b["sx"] for b in blocks]
    assert host(qx)[0].tolist() == sum((b["q"] for b in blocks), [])


@pytest.mark.parametrize("m,k,outliers", [(1, 32, False), (3, 96, True), (17, 288, True),
                                          (5, 2048, False), (512, 2048, True), (512, 8192, True),
                                          (16, 4096, True)])
def test_quantize_bit_exact(m, k, outliers):
    x, _, _ = inputs(100 + m, m, k, 64, outliers)
    qx, sx = w4.quantize_act(dev(x))
    q_ref, s_ref = oracle.quantize_activations(x)
    assert np.array_equal(host(qx), q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))


def test_quantize_special_values():
    g = np.random.default_rng(5)
    x = np.zeros((4, 256), dtype=np.float16)
    x[1] = (g.integers(-1023, 1024, 256) * 2.0 ** -24).astype(np.float16)   # fp16 subnormals
    x[2] = (g.integers(-254, 255, 256) / 2.0).astype(np.float16)             # many exact ties
    x[2, ::32] = 127.0
    x[3] = np.clip(g.standard_normal(256) * 2e4, -65504, 65504).astype(np.float16)  # up to the fp16 maximum
    x[3, 7] = 65504.0
    x[3, 64:96] = -0.0
    qx, sx = w4.quantize_act(dev(x))
    q_ref, s_ref = oracle.quantize_activations(x)
    assert np.array_equal(host(qx), q_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))


# -------------------------------------------------------------------- packer
@pytest.mark.parametrize("k,n", [(64, 64), (96, 192), (2048, 2560)])
def test_pack_bit_exact(k, n):
    _, qw, sw = inputs(7, 1, k, n)
    packed, ws = packed_on_gpu(qw, sw)
    p_ref, s_ref = oracle.pack_weights(qw, sw)
    assert np.array_equal(host(packed), p_ref)
    assert np.array_equal(host(ws).view(np.uint16), s_ref.view(np.uint16))


def test_pack_golden_layout():
    with open(os.path.join(GOLDEN, "pack_layout.json")) as f:
        d = json.load(f)
    qw = np.zeros((64, d["K"]), dtype=np.int8)          # N = 64: the library's minimum
    qw[: d["N"]] = np.array(d["qw"], dtype=np.int8)
    sw = np.ones((64, d["K"] // 32), dtype=np.float16)
    sw[: d["N"]] = np.array(d["sw"], dtype=np.float16)
    packed, ws = packed_on_gpu(qw, sw)
    p = host(packed)
    flat = [bytes(p[b, n]).hex() for b in range(d["K"] // 32) for n in range(d["N"])]
    assert flat == d["packed_hex"]
    assert host(ws)[:, : d["N"]].astype(np.float64).tolist() == d["w_scales"]


# --------------------------------------------------------------- block sums
TINY = [(1, 32, 64), (2, 64, 128), (3, 96, 192), (17, 288, 64), (4, 32 * 37, 320), (40, 1024, 640)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("m,k,n", TINY)
def test_block_sums_bit_exact(path, m, k, n):
    x, qw, sw = inputs(m * 1000 + k, m, k, n, outliers=True)
    packed, _ = packed_on_gpu(qw, sw)
    got = host(w4.block_sums(dev(x), packed, path=path))
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))


@pytest.mark.parametrize("path", PATHS)
def test_block_sums_extreme_values(path):
    """All codes at their extremes: |I| reaches 32 * 127 * 8 = 32512 in every block."""
    m, k, n = 2, 128, 64
    x = np.full((m, k), 3.0, dtype=np.float16)
    x[1] = -3.0
    qw = np.full((n, k), -8, dtype=np.int8)
    qw[1::2] = 7
    sw = np.ones((n, k // 32), dtype=np.float16)
    packed, _ = packed_on_gpu(qw, sw)
    got = host(w4.block_sums(dev(x), packed, path=path))
    assert got[0, 0, 0] == -32512 and got[1, 0, 0] == 32512
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))


@pytest.mark.parametrize("path", PATHS)
def test_block_sums_decode_shape(path):
    x, qw, sw = synth.workload_inputs("decode")["qkv"]
    packed, _ = packed_on_gpu(qw, sw)
    got = host(w4.block_sums(dev(x), packed, path=path))
    qx, _ = oracle.quantize_activations(x)
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))


# ----------------------------------------------------------------- linear
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("m,k,n", TINY)
def test_linear_tiny(path, m, k, n):
    x, qw, sw = inputs(m * 7 + k, m, k, n, outliers=True)
    packed, ws = packed_on_gpu(qw, sw)
    got = host(w4.linear(dev(x), packed, ws, path=path))
    assert_close(got, oracle.linear(x, qw, sw), f"path {path} M={m} K={k} N={n}")


def test_linear_golden_example():
    with open(os.path.join(GOLDEN, "linear_examples.json")) as f:
        d = json.load(f)
    x = np.array(d["x"], dtype=np.float16)
    qw = np.zeros((64, 64), dtype=np.int8)
    qw[:2] = np.array(d["qw"], dtype=np.int8)
    sw = np.ones((64, 2), dtype=np.float16)
    sw[:2] = np.array(d["sw"], dtype=np.float16)
    packed, ws = packed_on_gpu(qw, sw)
    for path in PATHS:
        got = host(w4.linear(dev(x), packed, ws, path=path))
        assert got[0, :2].tolist() == d["out"][0]      # exact: every term is a small dyadic number


@pytest.mark.parametrize("path", PATHS)
def test_linear_zero_input(path):
    x = np.zeros((3, 256), dtype=np.float16)
    _, qw, sw = inputs(3, 3, 256, 128)
    packed, ws = packed_on_gpu(qw, sw)
    got = host(w4.linear(dev(x), packed, ws, path=path))
    assert np.all(got == 0)


@pytest.mark.parametrize("path", PATHS)
def test_power_of_two_scaling_is_exact(path):
    """out(2 * sw) == 2 * out(sw) and out(4 * x) == 4 * out(x), bit for bit."""
    x, qw, sw = inputs(11, 5, 512, 256, outliers=True)
    packed, ws = packed_on_gpu(qw, sw)
    base = host(w4.linear(dev(x), packed, ws, path=path))
    packed2, ws2 = packed_on_gpu(qw, (sw.astype(np.float64) * 2).astype(np.float16))
    assert np.array_equal(host(w4.linear(dev(x), packed2, ws2, path=path)), 2 * base)
    x4 = (x.astype(np.float64) * 4).astype(np.float16)
    assert np.array_equal(host(w4.linear(dev(x4), packed, ws, path=path)), 4 * base)


@pytest.mark.parametrize("path", PATHS)
def test_repeat_runs_are_bit_identical(path):
    x, qw, sw = inputs(12, 6, 8192, 2048, outliers=True)     # split-K on both kernels
    packed, ws = packed_on_gpu(qw, sw)
    xd = dev(x)
    first = host(w4.linear(xd, packed, ws, path=path))
    for _ in range(3):
        assert np.array_equal(host(w4.linear(xd, packed, ws, path=path)), first)


@pytest.mark.parametrize("proj", list(synth.LAYER_SHAPES))
def test_decode_projection_full(proj):
    """Decode layer projections at M = 1 through the automatic stage choice, every output checked."""
    x, qw, sw = synth.workload_inputs("decode")[proj]
    packed, ws = packed_on_gpu(qw, sw)
    got = host(w4.linear(dev(x), packed, ws))
    assert_close(got, oracle.linear(x, qw, sw), proj)


def test_single_linear_full():
    x, qw, sw = synth.workload_inputs("single")["single"]
    packed, ws = packed_on_gpu(qw, sw)
    assert_close(host(w4.linear(dev(x), packed, ws)), oracle.linear(x, qw, sw), "single")


@pytest.mark.parametrize("proj", list(synth.LAYER_SHAPES))
def test_prefill_projection_sampled(proj):
    """Prefill projections at M = 512 (outlier channels) through the automatic stage choice;
    all rows of 256 seeded random columns checked against the oracle."""
    x, qw, sw = synth.workload_inputs("prefill")[proj]
    packed, ws = packed_on_gpu(qw, sw)
    got = host(w4.linear(dev(x), packed, ws))
    cols = np.sort(np.random.default_rng(0).choice(qw.shape[0], 256, replace=False))
    assert_close(got[:, cols], oracle.linear(x, qw[cols], sw[cols]), proj)


# One shape per GEMM tile plan: 128 x 32 (four waves along n), K split over four
# waves of one 32 x 32 tile (M <= 32, 32 < M <= 64 and M > 64), 128 x 64, eight-wave
# 128 x 128, and K split across workgroups (few tiles, long K) at both M ranges.
GEMM_PLANS = [(8, 64, 65536), (8, 96, 192), (40, 64, 65536), (40, 1024, 640), (130, 64, 32768),
              (130, 1024, 640), (8, 8192, 128), (130, 8192, 64)]


@pytest.mark.parametrize("m,k,n", GEMM_PLANS)
def test_gemm_every_tile_plan(m, k, n):
    x, qw, sw = inputs(m * 11 + k + n, m, k, n, outliers=True)
    packed, ws = packed_on_gpu(qw, sw)
    xd = dev(x)
    assert_close(host(w4.linear(xd, packed, ws, path=w4.PATH_GEMM)), oracle.linear(x, qw, sw),
                 f"GEMM M={m} K={k} N={n}")
    qx, _ = oracle.quantize_activations(x)
    got = host(w4.block_sums(xd, packed, path=w4.PATH_GEMM))
    assert np.array_equal(got.astype(np.int64), oracle.block_sums(qx, qw))


# One shape per GEMV launch plan: 64 columns in 512-thread workgroups (one chunk of K, and
# four), 64 columns in 256-thread workgroups, 8 columns in 512-thread workgroups (one chunk,
# two), 16 and 8 columns in 256-thread workgroups, and 32-column tiles of 4 and 8 rows.
GEMV_PLANS = [(1, 2048, 16384), (1, 8192, 16384), (1, 2048, 32768), (1, 8192, 2048), (1, 16384, 2048),
              (1, 2048, 8192), (1, 2048, 2560), (3, 4096, 16384), (8, 2048, 16384)]


@pytest.mark.parametrize("m,k,n", GEMV_PLANS)
def test_gemv_every_launch_plan(m, k, n):
    x, qw, sw = inputs(m * 13 + k + n, m, k, n, outliers=True)
    packed, ws = packed_on_gpu(qw, sw)
    assert_close(host(w4.linear(dev(x), packed, ws, path=w4.PATH_GEMV)), oracle.linear(x, qw, sw),
                 f"GEMV M={m} K={k} N={n}")


@pytest.mark.parametrize("m", synth.WORKLOADS["wide"]["M"])
def test_wide_linear_full(m):
    x, qw, sw = synth.workload_inputs("wide", m)["wide"]
    packed, ws = packed_on_gpu(qw, sw)
    xd = dev(x)
    ref = oracle.linear(x, qw, sw)
    for path in [w4.PATH_AUTO] + PATHS:
        assert_close(host(w4.linear(xd, packed, ws, path=path)), ref, f"wide M={m} path {path}")


# ------------------------------------------------------------------ argmax
def _check_argmax(x, qw, sw):
    packed, ws = packed_on_gpu(qw, sw)
    xd = dev(x)
    am, logits = w4.linear_argmax(xd, packed, ws, logits=True)
    am_only = w4.linear_argmax(xd, packed, ws)
    am, logits, am_only = host(am), host(logits), host(am_only)
    ref = oracle.linear(x, qw, sw)
    assert_close(logits, ref, "logits")
    assert np.array_equal(am, am_only)
    assert np.array_equal(am, oracle.argmax_first(logits))       # fused == argmax of own logits
    want = oracle.argmax_first(ref)
    for r in range(x.shape[0]):
        if am[r] != want[r]:     # allowed only for a near-tie within the output tolerance
            gap = ref[r, want[r]] - ref[r, am[r]]
            assert gap <= ATOL + RTOL * abs(ref[r, want[r]]), f"row {r}: {am[r]} vs {want[r]}"
    return am, want


def test_argmax_lm_head():
    """The LM head of the end-to-end workload: 2048 -> 262144, M = 1, every logit checked."""
    k, n = synth.LM_HEAD_SHAPE
    x, qw, sw = inputs(4, 1, k, n)
    am, want = _check_argmax(x, qw, sw)
    assert am[0] == want[0]


@pytest.mark.parametrize("m,k,n", [(1, 64, 64), (3, 96, 192), (9, 256, 4096), (64, 128, 640)])
def test_argmax_small(m, k, n):
    x, qw, sw = inputs(m + n, m, k, n, outliers=True)
    _check_argmax(x, qw, sw)


def test_argmax_ties_take_lowest_index():
    m, k, n = 2, 64, 256
    x, qw, sw = inputs(21, m, k, n)
    qw[200] = qw[37] = qw[130]          # identical columns give identical logits
    sw[200] = sw[37] = sw[130]
    qw[130] = np.where(qw[130] >= 0, 7, -8)
    packed, ws = packed_on_gpu(qw, sw)
    am, logits = w4.linear_argmax(dev(x), packed, ws, logits=True)
    logits, am = host(logits), host(am)
    assert np.all(logits[:, 37] == logits[:, 200])
    assert np.array_equal(am, oracle.argmax_first(logits))
    xz = np.zeros((m, k), dtype=np.float16)               # all logits are zero: index 0
    assert host(w4.linear_argmax(dev(xz), packed, ws)).tolist() == [0, 0]


def test_argmax_ties_at_the_row_maximum_across_workgroups():
    """Three identical weight columns in different workgroups of the LM head (1000, 70001 and
    200003: 64-column tiles) make the row maximum; the fused argmax returns the lowest of them."""
    k, n = synth.LM_HEAD_SHAPE
    x, qw, sw = inputs(23, 2, k, n)
    cols = [1000, 70001, 200003]
    q16 = oracle.quantize_activations(x)[0].astype(np.int64)
    best = np.where(q16[0] >= 0, 7, -8).astype(np.int8)     # row 0's codes all pull the same way
    for c in cols:
        qw[c] = best
        sw[c] = np.float16(0.02)
    packed, ws = packed_on_gpu(qw, sw)
    am, logits = w4.linear_argmax(dev(x), packed, ws, logits=True)
    am, logits = host(am), host(logits)
    assert logits[0, cols[0]] == logits[0, cols[1]] == logits[0, cols[2]] == logits[0].max()
    assert (logits[0] == logits[0].max()).sum() == 3
    assert am[0] == cols[0]
    assert np.array_equal(am, oracle.argmax_first(logits))
    # and the same logits when 1000 is taken out of the tie: the next lowest wins
    qw[1000] = 0
    packed, ws = packed_on_gpu(qw, sw)
    assert host(w4.linear_argmax(dev(x), packed, ws))[0] == cols[1]


def test_call_beyond_reserved_scratch_is_rejected():
    """A prefill linear whose staging exceeds the reserved scratch fails with W4A8_EINVAL before
    launching anything (out untouched) and runs after w4a8_reserve_scratch."""
    k, n = 8192, 64
    cap = w4.scratch_capacity()
    m = ((cap // (k + k // 8)) // 32 + 64) * 32
    need = w4.linear_scratch_bytes(m, k, n)
    assert need > cap
    x, qw, sw = inputs(25, m, k, n)
    packed, ws = packed_on_gpu(qw, sw)
    xd = dev(x)
    out = torch.full((m, n), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(w4.W4A8Error) as err:
        w4.linear(xd, packed, ws, out=out)
    assert err.value.code == w4.W4A8_EINVAL and "w4a8_reserve_scratch" in str(err.value)
    assert bool((host(out) == 7.0).all())
    w4.reserve_scratch(need)
    got = host(w4.linear(xd, packed, ws, out=out))
    rows = np.random.default_rng(26).choice(m, 64, replace=False)
    assert_close(got[rows], oracle.linear(x[rows], qw, sw), "sampled rows")


def test_argmax_back_to_back_calls():
    """The fused argmax leaves its slots reset: consecutive calls with different inputs agree
    with their own logits."""
    k, n = 512, 8192
    _, qw, sw = inputs(31, 1, k, n)
    packed, ws = packed_on_gpu(qw, sw)
    for s in range(5):
        x, _, _ = inputs(40 + s, 2, k, n)
        am, logits = w4.linear_argmax(dev(x), packed, ws, logits=True)
        assert np.array_equal(host(am), oracle.argmax_first(host(logits)))
