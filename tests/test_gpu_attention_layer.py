"""GPU parity of the decode layer with attention (w4a8_decoder_layer_attention) at the end-to-end
workload's shape: hidden 2048, 8 query heads of 256 over one KV head, qkv 2048 -> 2560, feed-forward
8192, an fp16 KV cache of the pages' context of 640 (ML Drift explainer on tech.dede.sh, section
"Stage-aware optimization for large language models") seeded for the 512 prompt positions.

Teacher-forced over three decode steps: each launch is checked on its own GPU inputs, which the
call leaves in its workspace -- qkv against the oracle linear (1e-3 + 1e-3 |ref|), the attention
output against the oracle attention of the GPU's own queries, key and value over the cache as the
call found it (half an fp16 ulp + 2^-12 sum_t p_t |V_t|), then o, gate/up, down and the residual
adds as in the one-token layer; the cache's new position holds fp16 of the key and value bit for bit."""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth
from oracle import attention as at

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
H, F = 2048, 8192
HQ, HKV, D = synth.ATTN_HEADS, synth.ATTN_KV_HEADS, synth.ATTN_HEAD_DIM
CAP = synth.CONTEXT
EPS, SCALE = 1e-6, 0.01


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, what):
    excess = np.abs(np.asarray(got, np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert (excess <= 0).all(), f"{what}: {(excess > 0).sum()} outside, max excess {excess.max():.3g}"


def test_decode_layer_with_attention_teacher_forced():
    w4.init(0)
    hw = synth.e2e_layer_weights(3)
    lw = {p: w4.Weights.pack(dev(q), dev(s)) for p, (q, s) in hw.items()}
    nq = lw["qkv"].N
    assert nq == (HQ + 2 * HKV) * D
    g = np.random.default_rng(77)
    prompt = synth.PREFILL_TOKENS
    k_past = g.standard_normal((HKV, prompt, D)).astype(np.float16)
    v_past = g.standard_normal((HKV, prompt, D)).astype(np.float16)
    kc, vc = w4.kv_cache(HKV, D, CAP)
    kc[:, :prompt] = dev(k_past)
    vc[:, :, :prompt] = dev(v_past.transpose(0, 2, 1))
    x = dev(synth.e2e_prompt()[-1:].astype(np.float32))
    ws = torch.zeros(w4.decoder_layer_workspace(1, H, lw["qkv"], lw["gate_up"]), dtype=torch.uint8, device=DEV)
    offs = w4.decoder_layer_workspace_offsets(1, H, lw["qkv"], lw["gate_up"])

    def region(wsb, name, dtype, count):
        return wsb[offs[name]:offs[name] + count * np.dtype(dtype).itemsize].view(dtype).reshape(1, count)

    for step in range(3):
        length = prompt + 1 + step
        x_in = host(x).copy()
        kc_in, vc_in = host(kc).copy(), host(vc).copy()
        w4.decoder_layer_attention(x, lw["qkv"], lw["o"], lw["gate_up"], lw["down"], SCALE, EPS, kc, vc, HQ, length, ws)
        wsb = host(ws)
        q = region(wsb, "q", np.float32, nq)
        a = region(wsb, "a", np.float16, H)
        o = region(wsb, "o", np.float32, H)
        gu = region(wsb, "g", np.float32, 2 * F)
        u = region(wsb, "u", np.float16, F)
        d = region(wsb, "d", np.float32, H)
        n1 = host(w4.residual_norm_cast(dev(x_in), eps=EPS))
        assert_close(q, oracle.linear(n1, *hw["qkv"]), f"step {step} qkv")
        # Attention on the GPU's own queries, key and value, over the cache as the call found it.
        qh = q[0, :HQ * D].reshape(HQ, D)
        k_new = q[0, HQ * D:(HQ + HKV) * D].reshape(HKV, D)
        v_new = q[0, (HQ + HKV) * D:].reshape(HKV, D)
        kp = kc_in[:, :length - 1]
        vp = vc_in[:, :, :length - 1].transpose(0, 2, 1)
        exact, mag = at.decode_attention_exact(qh, k_new, v_new, kp, vp)
        err = np.abs(a.reshape(HQ, D).astype(np.float64) - exact)
        bound = 0.5 * np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64) + 2.0 ** -12 * mag
        assert (err <= bound).all(), f"step {step} attention: {(err > bound).sum()} outside"
        kc_out, vc_out = host(kc), host(vc)
        assert np.array_equal(kc_out[:, length - 1], k_new.astype(np.float16))
        assert np.array_equal(vc_out[:, :, length - 1], v_new.astype(np.float16))
        assert np.array_equal(kc_out[:, :length - 1], kc_in[:, :length - 1])
        assert_close(o, oracle.linear(a, *hw["o"]), f"step {step} o")
        x_mid = oracle.residual_add(x_in, o, SCALE)
        n2 = host(w4.residual_norm_cast(dev(x_mid), eps=EPS))
        assert_close(gu, oracle.linear(n2, *hw["gate_up"]), f"step {step} gate_up")
        assert np.array_equal(u, oracle.gated_fp16(gu))
        assert_close(d, oracle.linear(u, *hw["down"]), f"step {step} down")
        assert np.array_equal(host(x), oracle.residual_add(x_mid, d, SCALE))
        print(f"step {step} (length {length}): every launch checked", flush=True)
    assert w4.take_device_errors() == 0


def test_attention_layer_from_o_in_one_launch_equals_three_gemvs():
    """With the resident layer available, w4a8_decoder_layer_attention runs o, gate/up and down
    as one launch of resident workgroups that starts from the attention output; it must leave
    the residual stream and every intermediate bit for bit as the three one-token GEMV
    launches do, over consecutive decode steps (each step's cache writes feed the next)."""
    h, hq, hkv, d = 2048, 8, 1, 256
    n_qkv, f, cap = (hq + 2 * hkv) * d, 8192, 640
    weights = {p: w4.Weights.pack(dev(synth.int4_values(synth.rng(71, i), n, k)),
                                  dev(synth.weight_scales(synth.rng(71, 10 + i), n, k)))
               for i, (p, (k, n)) in enumerate({"qkv": (h, n_qkv), "o": (h, h), "gate_up": (h, 2 * f),
                                                 "down": (f, h)}.items())}
    assert w4.layer_kernel(1, h, weights["qkv"], weights["gate_up"]) == w4.LAYER_RESIDENT
    g = np.random.default_rng(72)
    x0 = g.standard_normal((1, h)).astype(np.float32)
    kp = g.standard_normal((hkv, cap, d)).astype(np.float16)
    vp = g.standard_normal((hkv, d, cap)).astype(np.float16)
    results = {}
    for resident in (1, 0):
        w4.set_option(w4.OPTION_RESIDENT_LAYER, resident)
        try:
            x = dev(x0.copy())
            kc, vc = dev(kp.copy()), dev(vp.copy())
            ws = torch.zeros(w4.decoder_layer_workspace(1, h, weights["qkv"], weights["gate_up"]),
                             dtype=torch.uint8, device=DEV)
            steps = []
            for step in range(3):
                w4.decoder_layer_attention(x, weights["qkv"], weights["o"], weights["gate_up"], weights["down"],
                                           0.01, 1e-6, kc, vc, hq, 600 + step, ws)
                steps.append((host(x).copy(), host(ws).copy()))
            results[resident] = (steps, host(kc), host(vc))
        finally:
            w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)
    (one, k1, v1), (three, k3, v3) = results[1], results[0]
    for step, ((x1, ws1), (x3, ws3)) in enumerate(zip(one, three)):
        assert np.array_equal(x1.view(np.uint32), x3.view(np.uint32)), f"step {step}: residual stream"
        assert np.array_equal(ws1, ws3), f"step {step}: workspace intermediates"
    assert np.array_equal(k1.view(np.uint16), k3.view(np.uint16)) and np.array_equal(v1.view(np.uint16),
                                                                                       v3.view(np.uint16))
    assert w4.take_device_errors() == 0
