"""GPU parity of the decoder-layer glue, the layer chain and the LM-head argmax."""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EPS = 1e-6
SCALE = 0.01


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def fp16_ulp_diff(a16, b16):
    """Distance in fp16 units in the last place (same-sign finite values)."""
    ai = a16.view(np.int16).astype(np.int32)
    bi = b16.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -(ai & 0x7FFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFF), bi)
    return np.abs(ai - bi)


def test_residual_add_bit_exact():
    g = np.random.default_rng(0)
    x = (g.standard_normal((5, 2048)) * 3).astype(np.float32)
    d = (g.standard_normal((5, 2560)) * 50).astype(np.float32)
    xd = dev(x)
    w4.residual_norm_cast(xd, dev(d), alpha=SCALE, want_y=False)
    assert np.array_equal(host(xd), oracle.residual_add(x, d[:, :2048], SCALE))


@pytest.mark.parametrize("m,h", [(1, 2048), (7, 256), (512, 2048), (3, 96)])
def test_rms_norm_cast_within_one_ulp(m, h):
    g = np.random.default_rng(m + h)
    x = (g.standard_normal((m, h)) * g.uniform(0.1, 30, size=(m, 1))).astype(np.float32)
    y = host(w4.residual_norm_cast(dev(x), eps=EPS))
    ref = oracle.rms_norm_fp16(x, EPS)
    ulp = fp16_ulp_diff(y, ref)
    assert ulp.max() <= 1
    assert (ulp > 0).mean() < 0.01


def _weights(seed, h, n_qkv, f):
    shapes = {"qkv": (h, n_qkv), "o": (h, h), "gate_up": (h, 2 * f), "down": (f, h)}
    host_w, dev_w = {}, {}
    for i, (name, (k, n)) in enumerate(shapes.items()):
        qw = synth.int4_values(synth.rng(seed, 16 * i), n, k)
        sw = synth.weight_scales(synth.rng(seed, 16 * i + 1), n, k)
        host_w[name] = (qw, sw)
        dev_w[name] = w4.Weights.pack(dev(qw), dev(sw))
    return host_w, dev_w


def _run_layer(x, dev_w):
    m, h = x.shape
    ws = torch.empty(w4.decoder_layer_workspace(m, h, dev_w["qkv"], dev_w["gate_up"]), dtype=torch.uint8, device=DEV)
    xd = dev(x)
    w4.decoder_layer(xd, dev_w["qkv"], dev_w["o"], dev_w["gate_up"], dev_w["down"], SCALE, EPS, ws)
    return host(xd)


@pytest.mark.parametrize("m", [1, 3, 40, 130])
def test_decoder_layer_small(m):
    """Both stage kernels inside the layer chain, against the oracle chain from the same input."""
    h, n_qkv, f = 256, 320, 512
    host_w, dev_w = _weights(7, h, n_qkv, f)
    x = (np.random.default_rng(m).standard_normal((m, h)) * 2).astype(np.float32)
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    err = np.abs(got.astype(np.float64) - ref) - (1e-4 + 1e-4 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
    assert not np.array_equal(got, x)


@pytest.mark.parametrize("m", [200, 256])
def test_decoder_layer_gated_gemm_epilogue(m):
    """A gate/up GEMM wide enough for 128 x 128 tiles (2F = 32768) quantises fp16(gate * up)
    into the down projection's staging in its epilogue. At 200 rows the down projection's
    staging covers 224 rows (zero codes past row 200) against the gate/up tiles' 256, and the
    down projection splits K across workgroups with its staging outside library scratch."""
    h, n_qkv, f = 128, 192, 16384
    host_w, dev_w = _weights(21, h, n_qkv, f)
    x = (np.random.default_rng(m + 5).standard_normal((m, h)) * 2).astype(np.float32)
    assert w4.auto_path(m, h, 2 * f) == w4.PATH_GEMM and w4.auto_path(m, f, h) == w4.PATH_GEMM
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    # 16384-wide intermediates: a one-ulp fp16 difference in a normalised input can move an
    # int8 code by one, so the output tolerance itself applies (1e-3 abs + 1e-3 rel).
    err = np.abs(got.astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
    assert np.median(np.abs(got - ref)) < 1e-4
    assert not np.array_equal(got, x)


def test_decoder_layer_fused_epilogues_on_narrow_wide_grids():
    """22000 rows at hidden 192: the qkv GEMM (384 columns) runs 128 x 128 tiles, one of which
    quantises its first 64 columns (the end of the query slice) and writes the other 64; the
    gate/up GEMM (2F = 384) runs three 128-column tiles of 64 gate and 64 up columns each; the
    last 16 rows of every staging are padding."""
    h, n_qkv, f, m = 192, 384, 192, 22000
    host_w, dev_w = _weights(33, h, n_qkv, f)
    x = (np.random.default_rng(17).standard_normal((m, h)) * 2).astype(np.float32)
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    err = np.abs(got.astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
    assert np.median(np.abs(got - ref)) < 1e-4
    assert not np.array_equal(got, x)


def test_decoder_layer_full_decode_shape():
    """One layer at the end-to-end shapes (hidden 2048), M = 1."""
    h = 2048
    host_w, dev_w = _weights(4, h, 2560, 8192)
    x = synth.activations(synth.rng(4, 999), 1, h).astype(np.float32)
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    err = np.abs(got.astype(np.float64) - ref) - (1e-4 + 1e-4 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"


def test_decoder_layer_one_token_unfused_shape():
    """One token at a width whose gate/up tile cannot hold K = H in one GEMV chunk (64-column
    tiles cover 2048 of K): the layer falls back to the nine-launch chain."""
    h = 4096
    host_w, dev_w = _weights(8, h, h + 512, 16384)
    x = synth.activations(synth.rng(8, 999), 1, h).astype(np.float32)
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    # With 16384-wide intermediates a one-ulp fp16 difference in the normalised input can move an
    # int8 code by one, so this shape is held to the output tolerance itself (1e-3 abs + 1e-3 rel).
    err = np.abs(got.astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
    assert np.median(np.abs(got - ref)) < 1e-4


def test_decoder_layer_one_token_wide_workgroups():
    """One token at hidden 6144: the fused normalising kernels of the QKV and gate/up
    projections and the residual O projection run 8-column tiles in 512-thread workgroups."""
    h = 6144
    host_w, dev_w = _weights(9, h, h + 512, 2048)
    x = synth.activations(synth.rng(9, 999), 1, h).astype(np.float32)
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    err = np.abs(got.astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
    assert np.median(np.abs(got - ref)) < 1e-4


def test_chain_of_layers_and_lm_head_argmax():
    """Four layers and an LM head, GPU against oracle, no teacher forcing."""
    h, n_qkv, f, vocab = 256, 320, 512, 4096
    layers = [_weights(20 + i, h, n_qkv, f) for i in range(4)]
    qh = synth.int4_values(synth.rng(30, 0), vocab, h)
    sh = synth.weight_scales(synth.rng(30, 1), vocab, h)
    head = w4.Weights.pack(dev(qh), dev(sh))
    x = np.random.default_rng(5).standard_normal((2, h)).astype(np.float32)
    xd = dev(x)
    ws = torch.empty(w4.decoder_layer_workspace(2, h, layers[0][1]["qkv"], layers[0][1]["gate_up"]),
                     dtype=torch.uint8, device=DEV)
    xr = x.copy()
    for host_w, dev_w in layers:
        w4.decoder_layer(xd, dev_w["qkv"], dev_w["o"], dev_w["gate_up"], dev_w["down"], SCALE, EPS, ws)
        xr = oracle.decoder_layer(xr, host_w, SCALE, EPS)
    hd = w4.residual_norm_cast(xd, eps=EPS)
    am, logits = w4.linear_argmax(hd, head.packed, head.w_scales, logits=True)
    got_x, am, logits = host(xd), host(am), host(logits)
    assert np.abs(got_x - xr).max() <= 1e-3 * np.abs(xr).max()
    ref_logits = oracle.linear(oracle.rms_norm_fp16(xr, EPS), qh, sh)
    assert np.abs(logits - ref_logits).max() < 1e-2
    want = oracle.argmax_first(ref_logits)
    for r in range(2):
        if am[r] != want[r]:
            assert ref_logits[r, want[r]] - ref_logits[r, am[r]] < 1e-2, (am, want)
    # teacher-forced: the oracle on the GPU's own head input gives every logit within
    # 1e-3 + 1e-3 |ref| and the same index (the bound above covers four untethered layers)
    tf_logits = oracle.linear(host(hd), qh, sh)
    assert_close(logits, tf_logits, "teacher-forced logits")
    assert np.array_equal(am, oracle.argmax_first(tf_logits))


def assert_close(got, ref, what=""):
    excess = np.abs(np.asarray(got, np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    bad = int((excess > 0).sum())
    assert bad == 0, f"{what}: {bad} of {ref.size} outside 1e-3 + 1e-3 |ref|, max excess {excess.max():.3g}"


@pytest.mark.parametrize("m,h,vocab", [(1, 256, 4096), (1, 2048, 262144), (2, 256, 4096), (1, 8192, 4096),
                                        (1, 4096, 32768)])
def test_norm_linear_argmax(m, h, vocab):
    """LM-head argmax on the fp32 residual stream (one fused launch for one row; rows normalised
    first otherwise).  Teacher-forced: the oracle linear runs on the GPU's own fp16 head input
    (w4a8_residual_norm_cast, whose fp64 sum of squares gives the same fp16 values as the fused
    prologue), and every logit of both GPU paths is held to 1e-3 + 1e-3 |ref|."""
    qh = synth.int4_values(synth.rng(50 + h, 0), vocab, h)
    sh = synth.weight_scales(synth.rng(50 + h, 1), vocab, h)
    head = w4.Weights.pack(dev(qh), dev(sh))
    x = (np.random.default_rng(h + m).standard_normal((m, h)) * 3).astype(np.float32)
    am, logits = w4.norm_linear_argmax(dev(x), head.packed, head.w_scales, eps=EPS, logits=True)
    am, logits = host(am), host(logits)
    hb = host(w4.residual_norm_cast(dev(x), eps=EPS))
    assert fp16_ulp_diff(hb, oracle.rms_norm_fp16(x, EPS)).max() <= 1
    ref = oracle.linear(hb, qh, sh)
    assert_close(logits, ref, "logits")
    assert np.array_equal(am, oracle.argmax_first(logits))  # the fused argmax of its own logits
    want = oracle.argmax_first(ref)
    for r in range(m):
        if am[r] != want[r]:     # allowed only for a near-tie within the output tolerance
            assert ref[r, want[r]] - ref[r, am[r]] <= 1e-3 + 1e-3 * abs(ref[r, want[r]]), (am, want)
    # two-step path: the fp16 fused-argmax GEMV on the same fp16 values (its launch plan, and so
    # its fp32 summation order, may differ from the normalising kernel's)
    am2, logits2 = w4.linear_argmax(dev(hb), head.packed, head.w_scales, logits=True)
    am2, logits2 = host(am2), host(logits2)
    assert_close(logits2, ref, "two-step logits")
    assert np.array_equal(am2, oracle.argmax_first(logits2))


def test_graph_replay_matches_eager():
    """A captured token (2 layers + norm + fused argmax, and the one-launch normalising argmax)
    replays bit-identically to eager runs, with eager work and synchronisations between the replays."""
    h, n_qkv, f, vocab = 256, 320, 512, 2048
    layers = [_weights(40 + i, h, n_qkv, f)[1] for i in range(2)]
    qh = synth.int4_values(synth.rng(41, 0), vocab, h)
    sh = synth.weight_scales(synth.rng(41, 1), vocab, h)
    head = w4.Weights.pack(dev(qh), dev(sh))
    x0 = np.random.default_rng(6).standard_normal((1, h)).astype(np.float32)
    x = dev(x0)
    ws = torch.empty(w4.decoder_layer_workspace(1, h, layers[0]["qkv"], layers[0]["gate_up"]),
                     dtype=torch.uint8, device=DEV)
    hb = torch.empty((1, h), dtype=torch.float16, device=DEV)
    am = torch.empty((1,), dtype=torch.int32, device=DEV)
    am_fused = torch.empty((1,), dtype=torch.int32, device=DEV)

    def token():
        for lw in layers:
            w4.decoder_layer(x, lw["qkv"], lw["o"], lw["gate_up"], lw["down"], SCALE, EPS, ws)
        w4.residual_norm_cast(x, eps=EPS, y=hb)
        w4.linear_argmax(hb, head.packed, head.w_scales, argmax=am)
        w4.norm_linear_argmax(x, head.packed, head.w_scales, eps=EPS, argmax=am_fused)

    eager_x, eager_am, eager_fused = [], [], []
    x.copy_(dev(x0))
    for _ in range(3):
        token()
        eager_x.append(host(x).copy())
        eager_am.append(int(host(am)[0]))
        eager_fused.append(int(host(am_fused)[0]))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        token()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token()
    x.copy_(dev(x0))
    for i in range(3):
        graph.replay()
        assert np.array_equal(host(x), eager_x[i]), f"replay {i}"
        assert int(host(am)[0]) == eager_am[i], f"replay {i}"
        assert int(host(am_fused)[0]) == eager_fused[i], f"replay {i}"
        scratch = w4.linear(dev(np.ones((2, h), np.float16)), head.packed, head.w_scales)  # eager work between
        host(scratch)


def test_graph_of_a_prefill_layer_survives_scratch_growth():
    """A captured 130-row layer (prefill GEMMs staging in library scratch) keeps replaying
    correctly after w4a8_reserve_scratch has replaced the scratch it was captured with: the old
    buffer is retired, not freed, and eager calls between replays use the new one."""
    h, n_qkv, f, m = 256, 320, 512, 130
    _, dev_w = _weights(60, h, n_qkv, f)
    assert w4.decoder_layer_scratch_bytes(m, h, dev_w["qkv"], dev_w["gate_up"]) > 0
    x0 = np.random.default_rng(61).standard_normal((m, h)).astype(np.float32)
    x = dev(x0)
    ws = torch.empty(w4.decoder_layer_workspace(m, h, dev_w["qkv"], dev_w["gate_up"]), dtype=torch.uint8,
                     device=DEV)

    def layer():
        w4.decoder_layer(x, dev_w["qkv"], dev_w["o"], dev_w["gate_up"], dev_w["down"], SCALE, EPS, ws)

    eager = []
    for _ in range(3):
        layer()
        eager.append(host(x).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    before = w4.scratch_capacity()
    w4.reserve_scratch(before + (64 << 20))
    assert w4.scratch_capacity() >= before + (64 << 20)
    xe = np.random.default_rng(62).standard_normal((256, h)).astype(np.float16)
    x.copy_(dev(x0))
    for i in range(3):
        graph.replay()
        assert np.array_equal(host(x), eager[i]), f"replay {i}"
        # eager prefill work on the new scratch between replays
        host(w4.linear(dev(xe), dev_w["gate_up"].packed, dev_w["gate_up"].w_scales))


def test_residual_add_more_rows_than_a_grid_dimension():
    """The residual-only add walks rows with the grid's y stride: 70000 rows (more than the 65535
    a grid dimension holds), bit for bit against the oracle."""
    g = np.random.default_rng(11)
    x = (g.standard_normal((70000, 64)) * 3).astype(np.float32)
    d = (g.standard_normal((70000, 96)) * 50).astype(np.float32)
    xd = dev(x)
    w4.residual_norm_cast(xd, dev(d), alpha=SCALE, want_y=False)
    assert np.array_equal(host(xd), oracle.residual_add(x, d[:, :64], SCALE))


def test_decoder_layer_at_the_row_limit():
    """65536 rows (the layer's limit) through the prefill GEMMs and the glue kernels that quantise
    into GEMM staging, whose row loops cover more rows than one grid dimension holds."""
    h, n_qkv, f, m = 64, 128, 64, 65536
    host_w, dev_w = _weights(90, h, n_qkv, f)
    x = (np.random.default_rng(3).standard_normal((m, h)) * 2).astype(np.float32)
    assert w4.auto_path(m, h, 2 * f) == w4.PATH_GEMM
    got = _run_layer(x, dev_w)
    ref = oracle.decoder_layer(x, host_w, SCALE, EPS)
    err = np.abs(got.astype(np.float64) - ref) - (1e-4 + 1e-4 * np.abs(ref))
    assert err.max() <= 0, f"max excess {err.max():.3g}"
