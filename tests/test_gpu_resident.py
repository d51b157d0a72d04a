"""The one-token decoder layer in one launch (W4A8_LAYER_RESIDENT) on the GPU.

It must equal the four fused GEMV launches bit for bit: the residual stream
after the layer and every intermediate the layer leaves in its workspace (q,
a = fp16(q[:, :H]), o, g, u, d).  Checked at hidden 2048 / feed-forward 8192
for qkv widths 2048, 2560 and 4096 (256, 320 and 512 qkv tiles: workgroups
with one qkv tile, and with two), over chained calls (each call's output is
the next call's input, so the exchange epoch advances), under HIP graph
replay, and against the oracle on the GPU's own inputs.  The layer wiring is
the pages' decode step (ML Drift explainer on tech.dede.sh, section
"Stage-aware optimization for large language models").
"""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
H, F = 2048, 8192
EPS = 1e-6
SCALE = 0.01
SEED = 4242


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def weights(k, n, tid):
    qw = synth.int4_values(synth.rng(SEED, tid), n, k)
    sw = synth.weight_scales(synth.rng(SEED, tid + 1), n, k)
    return (qw, sw), w4.Weights.pack(dev(qw), dev(sw))


@pytest.fixture(scope="module")
def layer():
    w4.init(0)
    out = {"qkv": {}}
    for i, n in enumerate((2048, 2560, 4096)):
        out["qkv"][n] = weights(H, n, 10 + 2 * i)
    out["o"] = weights(H, H, 20)
    out["gate_up"] = weights(H, 2 * F, 22)
    out["down"] = weights(F, H, 24)
    return out


def stream_row(tid, outliers=True):
    g = synth.rng(SEED, tid)
    ch = synth.outlier_channels(synth.rng(SEED, tid + 1), H) if outliers else None
    return synth.activations(g, 1, H, ch).astype(np.float32)


def workspace(lay, n_qkv):
    qkv, gu = lay["qkv"][n_qkv][1], lay["gate_up"][1]
    nbytes = w4.decoder_layer_workspace(1, H, qkv, gu)
    return torch.zeros(nbytes, dtype=torch.uint8, device=DEV)


def run(x, lay, n_qkv, ws, resident):
    w4.set_option(w4.OPTION_RESIDENT_LAYER, 1 if resident else 0)
    try:
        w4.decoder_layer(x, lay["qkv"][n_qkv][1], lay["o"][1], lay["gate_up"][1], lay["down"][1], SCALE, EPS, ws)
    finally:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)


def regions(lay, n_qkv, wsb):
    """The intermediates the one-token layer writes, as host arrays of the workspace bytes."""
    offs = w4.decoder_layer_workspace_offsets(1, H, lay["qkv"][n_qkv][1], lay["gate_up"][1])
    sizes = {"q": (np.float32, n_qkv), "a": (np.float16, H), "o": (np.float32, H), "g": (np.float32, 2 * F),
             "u": (np.float16, F), "d": (np.float32, H)}
    return {k: wsb[offs[k]:offs[k] + n * np.dtype(t).itemsize].view(t).reshape(1, n) for k, (t, n) in sizes.items()}


def test_resident_kernel_selected(layer):
    qkv, gu = layer["qkv"][2560][1], layer["gate_up"][1]
    assert w4.layer_kernel(1, H, qkv, gu) == w4.LAYER_RESIDENT
    w4.set_option(w4.OPTION_RESIDENT_LAYER, 0)
    try:
        assert w4.layer_kernel(1, H, qkv, gu) == w4.LAYER_GEMV4
    finally:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)
    assert w4.layer_kernel(2, H, qkv, gu) != w4.LAYER_RESIDENT
    assert w4.take_device_errors() == 0


@pytest.mark.parametrize("n_qkv", [2560, 2048, 4096])
def test_resident_equals_four_launches(layer, n_qkv):
    """Three chained calls from an outlier row; every output and intermediate bit for bit."""
    x = dev(stream_row(100 + n_qkv))
    ws_r, ws_f = workspace(layer, n_qkv), workspace(layer, n_qkv)
    for step in range(3):
        xr, xf = x.clone(), x.clone()
        run(xr, layer, n_qkv, ws_r, resident=True)
        assert w4.take_device_errors() == 0, f"step {step}: a wait of the resident layer gave up"
        run(xf, layer, n_qkv, ws_f, resident=False)
        got, want = host(xr), host(xf)
        assert np.array_equal(got.view(np.int32), want.view(np.int32)), f"step {step}: residual stream differs"
        rr, rf = regions(layer, n_qkv, host(ws_r)), regions(layer, n_qkv, host(ws_f))
        for k in rr:
            assert np.array_equal(rr[k].view(np.uint8), rf[k].view(np.uint8)), f"step {step}: {k} differs"
        assert not np.array_equal(got, host(x))
        x = xr
        print(f"n_qkv {n_qkv} step {step}: equal to the four-launch layer", flush=True)


def test_resident_special_rows(layer):
    """An all-zero row (every block quantises to zero codes and scale 0) and a row with fp16-range
    outliers: still equal to the four launches bit for bit."""
    rows = [np.zeros((1, H), np.float32), stream_row(7) * np.float32(2000.0)]
    for r in rows:
        xr, xf = dev(r), dev(r)
        ws_r, ws_f = workspace(layer, 2560), workspace(layer, 2560)
        run(xr, layer, 2560, ws_r, resident=True)
        run(xf, layer, 2560, ws_f, resident=False)
        assert w4.take_device_errors() == 0
        assert np.array_equal(host(xr).view(np.int32), host(xf).view(np.int32))
        rr, rf = regions(layer, 2560, host(ws_r)), regions(layer, 2560, host(ws_f))
        for k in rr:
            assert np.array_equal(rr[k].view(np.uint8), rf[k].view(np.uint8)), k


def test_resident_layer_against_oracle(layer):
    """One call, every projection on the GPU's own inputs (teacher-forced) against the oracle."""
    x_in = stream_row(300)
    x = dev(x_in)
    ws = workspace(layer, 2560)
    run(x, layer, 2560, ws, resident=True)
    assert w4.take_device_errors() == 0
    r = regions(layer, 2560, host(ws))
    hw = {"qkv": layer["qkv"][2560][0], "o": layer["o"][0], "gate_up": layer["gate_up"][0], "down": layer["down"][0]}

    def close(got, ref, what):
        excess = np.abs(got.astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
        assert (excess <= 0).all(), f"{what}: max excess {excess.max():.3g}"

    n1 = host(w4.residual_norm_cast(dev(x_in), eps=EPS))
    close(r["q"], oracle.linear(n1, *hw["qkv"]), "qkv")
    assert np.array_equal(r["a"], r["q"][:, :H].astype(np.float16))
    close(r["o"], oracle.linear(r["a"], *hw["o"]), "o")
    x_mid = oracle.residual_add(x_in, r["o"], SCALE)
    n2 = host(w4.residual_norm_cast(dev(x_mid), eps=EPS))
    close(r["g"], oracle.linear(n2, *hw["gate_up"]), "gate_up")
    assert np.array_equal(r["u"], oracle.gated_fp16(r["g"]))
    close(r["d"], oracle.linear(r["u"], *hw["down"]), "down")
    assert np.array_equal(host(x), oracle.residual_add(x_mid, r["d"], SCALE))


def test_resident_layer_graph_replay(layer):
    """Four resident calls captured in a HIP graph: every replay equals the eager chain."""
    x0 = stream_row(500)
    ws = workspace(layer, 2560)
    ref = dev(x0)
    for _ in range(4):
        run(ref, layer, 2560, ws, resident=True)
    want = host(ref)
    x = dev(x0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(x, layer, 2560, ws, resident=True)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(4):
            run(x, layer, 2560, ws, resident=True)
    for rep in range(3):
        x.copy_(dev(x0))
        graph.replay()
        assert np.array_equal(host(x).view(np.int32), want.view(np.int32)), f"replay {rep}"
        eager = dev(x0)
        run(eager, layer, 2560, ws, resident=True)  # eager work between the replays
        torch.cuda.synchronize()
    assert w4.take_device_errors() == 0


def test_resident_many_calls(layer):
    """Sixty-four back-to-back calls (the epoch advances every call): no wait gives up and the
    result equals the same chain on the four launches."""
    x0 = stream_row(900)
    xr, xf = dev(x0), dev(x0)
    ws = workspace(layer, 2560)
    for _ in range(64):
        run(xr, layer, 2560, ws, resident=True)
    assert w4.take_device_errors() == 0
    for _ in range(64):
        run(xf, layer, 2560, ws, resident=False)
    assert np.array_equal(host(xr).view(np.int32), host(xf).view(np.int32))


@pytest.fixture(scope="module")
def stack_layers(layer):
    """Five distinct layers (qkv width 2560); longer stacks repeat them cyclically."""
    out = [{"qkv": layer["qkv"][2560][1], "o": layer["o"][1], "gate_up": layer["gate_up"][1],
            "down": layer["down"][1]}]
    for i in range(1, 5):
        out.append({"qkv": weights(H, 2560, 100 + 8 * i)[1], "o": weights(H, H, 102 + 8 * i)[1],
                    "gate_up": weights(H, 2 * F, 104 + 8 * i)[1], "down": weights(F, H, 106 + 8 * i)[1]})
    return out


def run_single(x, lw, ws, resident):
    w4.set_option(w4.OPTION_RESIDENT_LAYER, 1 if resident else 0)
    try:
        w4.decoder_layer(x, lw["qkv"], lw["o"], lw["gate_up"], lw["down"], SCALE, EPS, ws)
    finally:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)


@pytest.mark.parametrize("n", [1, 2, 5, 33])
def test_stack_equals_layer_by_layer(layer, stack_layers, n):
    """A stack of n layers in one launch (two launches for 33) equals n one-launch layers and n
    four-launch layers bit for bit, and leaves the last layer's intermediates in the workspace."""
    lays = [stack_layers[i % len(stack_layers)] for i in range(n)]
    x0 = stream_row(700 + n)
    xs, xr, xf = dev(x0), dev(x0), dev(x0)
    ws_s, ws_r, ws_f = workspace(layer, 2560), workspace(layer, 2560), workspace(layer, 2560)
    w4.decoder_stack(xs, lays, SCALE, EPS, ws_s)
    assert w4.take_device_errors() == 0
    for lw in lays:
        run_single(xr, lw, ws_r, resident=True)
    for lw in lays:
        run_single(xf, lw, ws_f, resident=False)
    got = host(xs)
    assert np.array_equal(got.view(np.int32), host(xr).view(np.int32)), "stack vs one-launch layers"
    assert np.array_equal(got.view(np.int32), host(xf).view(np.int32)), "stack vs four-launch layers"
    rs, rf = regions(layer, 2560, host(ws_s)), regions(layer, 2560, host(ws_f))
    for k in rs:
        assert np.array_equal(rs[k].view(np.uint8), rf[k].view(np.uint8)), f"last layer's {k}"
    print(f"stack of {n}: equal to layer-by-layer", flush=True)


def test_stack_four_launch_fallback(layer, stack_layers):
    """With the one-launch kernel switched off, the stack runs layer by layer on the four launches."""
    lays = stack_layers[:3]
    x0 = stream_row(811)
    xs, xf = dev(x0), dev(x0)
    ws = workspace(layer, 2560)
    w4.set_option(w4.OPTION_RESIDENT_LAYER, 0)
    try:
        w4.decoder_stack(xs, lays, SCALE, EPS, ws)
        for lw in lays:
            w4.decoder_layer(xf, lw["qkv"], lw["o"], lw["gate_up"], lw["down"], SCALE, EPS, ws)
    finally:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)
    assert np.array_equal(host(xs).view(np.int32), host(xf).view(np.int32))


def test_stack_graph_replay(layer, stack_layers):
    """A 26-layer stack captured in a HIP graph: every replay equals the eager stack."""
    lays = [stack_layers[i % len(stack_layers)] for i in range(26)]
    x0 = stream_row(900)
    ws = workspace(layer, 2560)
    ref = dev(x0)
    w4.decoder_stack(ref, lays, SCALE, EPS, ws)
    want = host(ref)
    x = dev(x0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w4.decoder_stack(x, lays, SCALE, EPS, ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w4.decoder_stack(x, lays, SCALE, EPS, ws)
    for rep in range(3):
        x.copy_(dev(x0))
        graph.replay()
        assert np.array_equal(host(x).view(np.int32), want.view(np.int32)), f"replay {rep}"
        eager = dev(x0)
        w4.decoder_stack(eager, lays[:2], SCALE, EPS, ws)  # other eager work between the replays
        torch.cuda.synchronize()
    assert w4.take_device_errors() == 0
