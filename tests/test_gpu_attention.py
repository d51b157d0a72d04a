"""GPU parity of decode attention (w4a8_decode_attention) against oracle/attention.py.

Bar: every output within half an fp16 ulp of the oracle's unrounded fp64 result, plus
2^-12 * sum_t p_t |V_t|.  The kernel rounds an fp32 result once to fp16.  The fp32
score of n = head_dim products carries a relative error of about n * 2^-24 of
sum |q k| / sqrt(D) (about 2^-16 of it for D = 256), and that error reaches each
weight p_t as a relative error.  The last term therefore bounds the error the
result carries into the rounding, with margin.  The cache update is checked bit for
bit.  Unwritten cache slots are filled with NaN and Inf bit patterns: the kernel
reads them and must not let them through."""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
from oracle import attention as at
from synth import ATTN_HEAD_DIM, ATTN_HEADS, ATTN_KV_HEADS, CONTEXT, PREFILL_TOKENS, attention_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def garbage_bits(g, shape):
    """fp16 bit patterns: random, with one in four a NaN or an infinity."""
    bits = g.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    special = g.random(shape) < 0.25
    bits[special] = g.choice(np.array([0x7C00, 0xFC00, 0x7E00, 0xFFFF], np.uint16), size=int(special.sum()))
    return bits


def build_caches(k_past, v_past, capacity, seed):
    """Library storage of the logical past keys/values, slots from length-1 on filled with garbage."""
    hkv, lp, d = k_past.shape
    g = np.random.default_rng(seed)
    kc = garbage_bits(g, (hkv, capacity, d))
    vc = garbage_bits(g, (hkv, d, capacity))
    kc[:, :lp] = k_past.view(np.uint16)
    vc[:, :, :lp] = v_past.view(np.uint16).transpose(0, 2, 1)
    return kc, vc


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ulp16(x):
    return np.spacing(np.abs(x).astype(np.float16)).astype(np.float64)


def check(got, exact, mag, what):
    got = got.astype(np.float64)
    bound = 0.5 * ulp16(exact) + 2.0 ** -12 * mag
    err = np.abs(got - exact)
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} outside, worst {np.max(err - bound):.3g}"


def run(q, k_new, v_new, k_past, v_past, capacity, seed=0):
    hkv, d = k_new.shape
    length = k_past.shape[1] + 1
    kc, vc = build_caches(k_past, v_past, capacity, seed)
    kd, vd = to_dev(kc.view(np.float16)), to_dev(vc.view(np.float16))
    out = w4.decode_attention(to_dev(q), to_dev(k_new), to_dev(v_new), kd, vd, length)
    torch.cuda.synchronize()
    kc_exp, vc_exp = kc.copy(), vc.copy()
    kc_exp[:, length - 1] = k_new.astype(np.float16).view(np.uint16)
    vc_exp[:, :, length - 1] = v_new.astype(np.float16).view(np.uint16)
    assert np.array_equal(kd.cpu().numpy().view(np.uint16), kc_exp)
    assert np.array_equal(vd.cpu().numpy().view(np.uint16), vc_exp)
    return out.cpu().numpy()


# (Hq, Hkv, D, length, capacity): the layer's 8 x 256 heads over one KV head at the pages'
# context of 640 and at the first decode step after the 512-token prefill; one chunk,
# one position, a chunk plus one; grouped, multi-head and odd group sizes; long contexts
# whose chunk partials are merged in two levels.
CASES = [
    (ATTN_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM, CONTEXT, CONTEXT),
    (ATTN_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM, PREFILL_TOKENS + 1, CONTEXT),
    (8, 1, 256, 64, 64),
    (8, 1, 256, 1, 64),
    (8, 1, 256, 65, 128),
    (8, 1, 256, 300, 320),        # flagged-word merge with two outputs per thread (5 chunks, 4 merging)
    (8, 1, 256, 1024, 1024),      # flagged-word merge over two chunk ranges per output (16 chunks)
    (4, 2, 128, 300, 320),
    (6, 3, 64, 100, 128),
    (3, 3, 64, 77, 128),
    (8, 8, 128, 200, 256),
    (5, 1, 64, 1000, 1024),
    (16, 2, 256, 2048, 2112),
    (4, 2, 128, 5000, 5056),      # five merge groups of unequal size (4 x 16 + 15 chunks)
    (8, 1, 256, 32768, 32768),    # 32 merge groups of 16 chunks
    (4096, 4096, 64, 40, 64),     # the most KV heads: fewer merge groups per head fit the tickets
    (2048, 2048, 64, 1040, 1088), # 2048 KV heads of two merge groups (16 + 1 chunks), ticket stride 31
]


@pytest.mark.parametrize("hq,hkv,d,length,cap", CASES)
def test_decode_attention(hq, hkv, d, length, cap):
    seed = hq * 7919 + hkv * 104729 + d + length
    q, k_new, v_new, k_past, v_past = attention_inputs(seed, hq, hkv, d, length)
    got = run(q, k_new, v_new, k_past, v_past, cap, seed)
    exact, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    check(got, exact, mag, f"Hq={hq} Hkv={hkv} D={d} L={length}")
    # The fp32 error is far below the fp16 rounding step, so nearly every output rounds
    # as the oracle's does (measured on MI355X: 99.5 % to 100 % per case).
    same = np.mean(got == at.decode_attention(q, k_new, v_new, k_past, v_past))
    print(f"Hq={hq} Hkv={hkv} D={d} L={length}: {same:.4f} of outputs equal the oracle's fp16")
    assert same >= 0.99


@pytest.mark.parametrize("gain", [0.0, 8.0, 40.0])
def test_decode_attention_score_spread(gain):
    """Uniform weights (zero query), sharp weights and near one-hot weights."""
    q, k_new, v_new, k_past, v_past = attention_inputs(11, 8, 1, 256, 600, q_gain=gain)
    got = run(q, k_new, v_new, k_past, v_past, 640, 11)
    exact, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    check(got, exact, mag, f"q gain {gain}")


def test_decode_steps_carry_the_cache():
    """Eight decode steps from position 512: each call appends its token to the caches the
    next call reads (nothing re-uploaded), checked against the oracle step by step."""
    hq, hkv, d, cap = ATTN_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM, CONTEXT
    q, _, _, k_past, v_past = attention_inputs(21, hq, hkv, d, PREFILL_TOKENS + 1)
    kc, vc = build_caches(k_past, v_past, cap, 21)
    kd, vd = to_dev(kc.view(np.float16)), to_dev(vc.view(np.float16))
    g = np.random.default_rng(22)
    for step in range(8):
        length = PREFILL_TOKENS + 1 + step
        q = (g.standard_normal((hq, d)) * 2).astype(np.float32)
        k_new = g.standard_normal((hkv, d)).astype(np.float32)
        v_new = g.standard_normal((hkv, d)).astype(np.float32)
        got = w4.decode_attention(to_dev(q), to_dev(k_new), to_dev(v_new), kd, vd, length).cpu().numpy()
        exact, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
        check(got, exact, mag, f"step {step}")
        k_past = np.concatenate([k_past, k_new.astype(np.float16)[:, None]], axis=1)
        v_past = np.concatenate([v_past, v_new.astype(np.float16)[:, None]], axis=1)


def test_decode_attention_repeat_bit_identical():
    q, k_new, v_new, k_past, v_past = attention_inputs(31, 8, 1, 256, 640)
    kc, vc = build_caches(k_past, v_past, 640, 31)
    kd, vd = to_dev(kc.view(np.float16)), to_dev(vc.view(np.float16))
    args = (to_dev(q), to_dev(k_new), to_dev(v_new), kd, vd, 640)
    first = w4.decode_attention(*args).cpu().numpy()
    for _ in range(3):
        assert np.array_equal(w4.decode_attention(*args).cpu().numpy(), first)


def test_decode_attention_reads_qkv_row_slices():
    """q, k_new and v_new as views of one fp32 QKV output row [2560] (8 x 256 + 256 + 256)."""
    q, k_new, v_new, k_past, v_past = attention_inputs(41, 8, 1, 256, 600)
    row = to_dev(np.concatenate([q.reshape(-1), k_new.reshape(-1), v_new.reshape(-1)]))
    kc, vc = build_caches(k_past, v_past, 640, 41)
    kd, vd = to_dev(kc.view(np.float16)), to_dev(vc.view(np.float16))
    got = w4.decode_attention(row[:2048].view(8, 256), row[2048:2304].view(1, 256), row[2304:].view(1, 256),
                              kd, vd, 600).cpu().numpy()
    exact, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
    check(got, exact, mag, "QKV row slices")


def test_flagged_merge_regions_across_shapes():
    """Calls of different shapes alternate on the flagged-word merge (at most 32 chunks, at
    most 16 KV heads): each KV head keeps its own region of flagged words, so a word an
    earlier call of another shape left behind never passes for the current call's.  (A
    layout indexed by the call's shape failed exactly this: a three-head call after a
    one-head call read head 1's words from the earlier call's head 0.)"""
    shapes = [(8, 1, 256, 640, 640), (3, 3, 64, 77, 128), (8, 8, 128, 200, 256), (8, 1, 256, 64, 64),
              (6, 3, 64, 100, 128), (16, 2, 256, 2048, 2112), (3, 3, 64, 77, 128), (8, 1, 256, 640, 640)]
    for i, (hq, hkv, d, length, cap) in enumerate(shapes):
        q, k_new, v_new, k_past, v_past = attention_inputs(500 + i, hq, hkv, d, length)
        got = run(q, k_new, v_new, k_past, v_past, cap, 500 + i)
        exact, mag = at.decode_attention_exact(q, k_new, v_new, k_past, v_past)
        check(got, exact, mag, f"call {i}: Hq={hq} Hkv={hkv} D={d} L={length}")
    assert w4.take_device_errors() == 0
