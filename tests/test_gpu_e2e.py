"""GPU parity at the shapes the benchmark times.

* The prefill decoder layer of the end-to-end workload: hidden 2048, 512 token
  rows with outlier channels, six launches (prefill GEMMs whose epilogues
  quantise into the next GEMM's staging and add into the residual stream).
  It must equal the chain of separate calls bit for bit, and each step of
  that chain is checked on its own GPU inputs over every row and column.  A
  check of the layer output alone against the oracle layer cannot hold the
  stated tolerance at this shape: a one-unit fp16 difference in an
  intermediate (within tolerance) can move an int8 code of a 32-element block
  whose scale the x20 outlier channels have made large, and the next
  projection multiplies that step by its weights.
* The end-to-end decode: 26 layers at hidden 2048 and the 2048 -> 262144 LM
  head with the fused argmax, entered from the last row of the 512-token
  prefill (the pages' benchmark: prefill 512 / decode 128 with argmax
  sampling, ML Drift explainer on tech.dede.sh, section "Stage-aware
  optimization for large language models").  Teacher-forced: every
  projection of every layer is checked on the GPU's own inputs, which the
  one-token layer leaves in its workspace, and the head's logits on the GPU's
  own fp16 head input.

fp32 projection outputs are held to |gpu - ref| <= 1e-3 + 1e-3 |ref| against
the fp64 oracle; fp16 casts, gated products, residual adds and argmax indices
bit for bit.
"""
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
H = synth.LAYER_SHAPES["o"][0]
N_QKV = synth.LAYER_SHAPES["qkv"][1]
F = synth.LAYER_SHAPES["down"][0]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, what):
    excess = np.abs(np.asarray(got, np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    bad = int((excess > 0).sum())
    assert bad == 0, f"{what}: {bad} of {ref.size} outside 1e-3 + 1e-3 |ref|, max excess {excess.max():.3g}"


def pack_layer(host_w):
    return {p: w4.Weights.pack(dev(qw), dev(sw)) for p, (qw, sw) in host_w.items()}


def run_layer(x, dev_w, ws):
    w4.decoder_layer(x, dev_w["qkv"], dev_w["o"], dev_w["gate_up"], dev_w["down"], SCALE, EPS, ws)


def workspace(m, dev_w):
    return torch.empty(w4.decoder_layer_workspace(m, H, dev_w["qkv"], dev_w["gate_up"]), dtype=torch.uint8,
                       device=DEV)


def oracle_linear_rows(x16, qw, sw, chunk=64):
    """oracle.linear over row chunks (its integer block sums of 512 rows would not fit memory)."""
    return np.concatenate([oracle.linear(x16[i:i + chunk], qw, sw) for i in range(0, x16.shape[0], chunk)])


def chain(x, dev_w):
    """The layer as separate calls (norm, linears on the prefill GEMM, residual adds) on a copy of
    the GPU stream x, with the casts formed on the host by the oracle's own definitions.  Returns
    the output and every intermediate, each the input of the next step."""
    xc = x.clone()
    t = {"x": host(xc).copy()}
    n1 = w4.residual_norm_cast(xc, eps=EPS)
    t["n1"] = host(n1)
    q = w4.linear(n1, dev_w["qkv"].packed, dev_w["qkv"].w_scales, path=w4.PATH_GEMM)
    t["q"] = host(q)
    t["a"] = t["q"][:, :H].astype(np.float16)
    o = w4.linear(dev(t["a"]), dev_w["o"].packed, dev_w["o"].w_scales, path=w4.PATH_GEMM)
    t["o"] = host(o)
    n2 = w4.residual_norm_cast(xc, o, alpha=SCALE, eps=EPS)
    t["x_mid"], t["n2"] = host(xc).copy(), host(n2)
    g = w4.linear(n2, dev_w["gate_up"].packed, dev_w["gate_up"].w_scales, path=w4.PATH_GEMM)
    t["g"] = host(g)
    t["u"] = oracle.gated_fp16(t["g"])
    d = w4.linear(dev(t["u"]), dev_w["down"].packed, dev_w["down"].w_scales, path=w4.PATH_GEMM)
    t["d"] = host(d)
    w4.residual_norm_cast(xc, d, alpha=SCALE, eps=EPS, want_y=False)
    t["out"] = host(xc)
    return t


def check_chain(t, host_w, rows):
    """Every step of the chain on its own GPU inputs, for the given rows."""
    x = t["x"][rows]
    assert fp16_ulp_diff(t["n1"][rows], oracle.rms_norm_fp16(x, EPS)).max() <= 1
    assert_close(t["q"][rows], oracle_linear_rows(t["n1"][rows], *host_w["qkv"]), "qkv")
    assert_close(t["o"][rows], oracle_linear_rows(t["a"][rows], *host_w["o"]), "o")
    assert np.array_equal(t["x_mid"][rows], oracle.residual_add(x, t["o"][rows], SCALE))
    assert fp16_ulp_diff(t["n2"][rows], oracle.rms_norm_fp16(t["x_mid"][rows], EPS)).max() <= 1
    assert_close(t["g"][rows], oracle_linear_rows(t["n2"][rows], *host_w["gate_up"]), "gate_up")
    assert_close(t["d"][rows], oracle_linear_rows(t["u"][rows], *host_w["down"]), "down")
    assert np.array_equal(t["out"][rows], oracle.residual_add(t["x_mid"][rows], t["d"][rows], SCALE))


def fp16_ulp_diff(a16, b16):
    ai = a16.view(np.int16).astype(np.int32)
    bi = b16.view(np.int16).astype(np.int32)
    ai = np.where(ai < 0, -(ai & 0x7FFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFF), bi)
    return np.abs(ai - bi)


def test_prefill_layer_at_full_shape():
    """Layer 0 of the end-to-end workload on its 512-token prompt (outlier channels x20).  The
    six-launch prefill path (norms quantised into GEMM staging, the query-slice cast and the gated
    product quantised in GEMM epilogues, residual adds in GEMM epilogues) equals the chain of
    separate calls bit for bit, and every step of that chain, all 512 rows and every column,
    matches the oracle on its own GPU inputs."""
    m = synth.PREFILL_TOKENS
    host_w = synth.e2e_layer_weights(0)
    dev_w = pack_layer(host_w)
    for k, n in [(H, N_QKV), (H, H), (H, 2 * F), (F, H)]:
        assert w4.auto_path(m, k, n) == w4.PATH_GEMM
    x = synth.e2e_prompt().astype(np.float32)
    xd = dev(x)
    t = chain(xd, dev_w)
    run_layer(xd, dev_w, workspace(m, dev_w))
    got = host(xd)
    assert np.array_equal(got, t["out"])
    assert not np.array_equal(got, x)
    check_chain(t, host_w, np.arange(m))


def check_one_token_layer(x_in, x_out, wsb, offs, host_w):
    """Every projection of a one-token layer on the GPU's own inputs."""
    def region(name, dtype, count):
        start = offs[name]
        return wsb[start:start + count * np.dtype(dtype).itemsize].view(dtype).reshape(1, count)

    q = region("q", np.float32, N_QKV)
    a = region("a", np.float16, H)
    o = region("o", np.float32, H)
    g = region("g", np.float32, 2 * F)
    u = region("u", np.float16, F)
    d = region("d", np.float32, H)
    # The GPU's fp16 input of qkv: the glue kernel forms the same values as the fused prologue.
    n1 = host(w4.residual_norm_cast(dev(x_in), eps=EPS))
    assert_close(q, oracle.linear(n1, *host_w["qkv"]), "qkv")
    assert np.array_equal(a, q[:, :H].astype(np.float16))
    assert_close(o, oracle.linear(a, *host_w["o"]), "o")
    x_mid = oracle.residual_add(x_in, o, SCALE)
    n2 = host(w4.residual_norm_cast(dev(x_mid), eps=EPS))
    assert_close(g, oracle.linear(n2, *host_w["gate_up"]), "gate_up")
    assert np.array_equal(u, oracle.gated_fp16(g))
    assert_close(d, oracle.linear(u, *host_w["down"]), "down")
    assert np.array_equal(x_out, oracle.residual_add(x_mid, d, SCALE))


def test_end_to_end_decode_teacher_forced():
    """The 26-layer prefill of 512 rows (each layer equal to the chain of separate calls bit for
    bit, and that chain checked step by step on five rows, the last among them), then three
    decode steps from the last row: each layer's q, a, o, g, u, d and output on the GPU's own
    inputs, and the LM head's 262144 logits and argmax on the GPU's own fp16 head input."""
    n_layers = synth.N_LAYERS_E2E
    host_layers = [synth.e2e_layer_weights(i) for i in range(n_layers)]
    dev_layers = [pack_layer(hw) for hw in host_layers]
    qh, sh = synth.e2e_head_weights()
    head = w4.Weights.pack(dev(qh), dev(sh))
    print(f"weights of {n_layers} layers and the head packed", flush=True)

    m = synth.PREFILL_TOKENS
    x = dev(synth.e2e_prompt().astype(np.float32))
    ws = workspace(m, dev_layers[0])
    rows = [0, 137, 300, 402, m - 1]
    for i in range(n_layers):
        t = chain(x, dev_layers[i])
        run_layer(x, dev_layers[i], ws)
        assert np.array_equal(host(x), t["out"]), f"prefill layer {i}"
        check_chain(t, host_layers[i], rows)
    print("prefill checked", flush=True)

    xd = x[m - 1:m].clone()
    ws1 = workspace(1, dev_layers[0])
    offs = w4.decoder_layer_workspace_offsets(1, H, dev_layers[0]["qkv"], dev_layers[0]["gate_up"])
    ids = []
    for step in range(3):
        for i in range(n_layers):
            x_in = host(xd).copy()
            run_layer(xd, dev_layers[i], ws1)
            check_one_token_layer(x_in, host(xd), host(ws1), offs, host_layers[i])
        am, logits = w4.norm_linear_argmax(xd, head.packed, head.w_scales, eps=EPS, logits=True)
        am, logits = host(am), host(logits)
        hb = host(w4.residual_norm_cast(xd, eps=EPS))
        ref = oracle.linear(hb, qh, sh)
        assert_close(logits, ref, f"step {step} head")
        assert np.array_equal(am, oracle.argmax_first(logits))
        want = oracle.argmax_first(ref)
        if am[0] != want[0]:     # allowed only for a near-tie within the output tolerance
            assert ref[0, want[0]] - ref[0, am[0]] <= 1e-3 + 1e-3 * abs(ref[0, want[0]])
        ids.append(int(am[0]))
        print(f"decode step {step}: 26 layers and the head checked, id {ids[-1]}", flush=True)
