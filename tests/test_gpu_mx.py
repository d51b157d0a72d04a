"""GPU parity of the MX variant: MXFP8 activation conversion and MXFP4 weight packing
bit for bit against oracle/mx.py; the block-scaled GEMM within
1e-3 + 1e-3 |ref| + 2^-12 sum_k |a_k w_k|.

The last term is the instruction's own rounding: v_mfma_scale_f32_32x32x64_f8f6f4
sums the 64 scaled products of each K step in an internal format narrower than
fp32 (measured on gfx950: errors up to 5.4e-5 of sum |a w| where fp32 would give
about 1e-7), so an output that is a small difference of large terms carries an
absolute error proportional to the terms, not to the result."""
import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
from oracle import mx

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL = 1e-3
RTOL = 1e-3


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def activations(seed, m, k):
    """N(0, 1) fp16 rows with per-row magnitudes over many binades, 1% outlier channels x20,
    an all-zero block and fp16 subnormals."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)) * np.exp2(g.integers(-10, 6, size=(m, 1)))
    ch = g.choice(k, max(1, k // 100), replace=False)
    x[:, ch] *= 20
    x[0, :32] = 0.0
    if k >= 96:
        x[-1, 64:96] = g.standard_normal(32) * 2.0 ** -20     # subnormal fp16 range
    return x.astype(np.float16)


def weights(seed, n, k):
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)) * 0.02 * np.exp2(g.integers(-3, 3, size=(n, k // 32))).repeat(32, axis=1)
    w[-1, :32] = 0.0
    return w.astype(np.float16)


@pytest.mark.parametrize("m,k", [(1, 64), (3, 128), (130, 2048), (17, 8192)])
def test_mx_quantize_act_bit_exact(m, k):
    x = activations(m + k, m, k)
    codes, scales = w4.mx_quantize_act(dev(x))
    ref_c, ref_s = mx.mx_quantize(x, "e4m3")
    assert np.array_equal(host(scales), ref_s.T)
    assert np.array_equal(host(codes), ref_c.reshape(m, k // 32, 32).transpose(1, 0, 2))


@pytest.mark.parametrize("n,k", [(64, 64), (192, 256), (2560, 2048)])
def test_mx_pack_bit_exact(n, k):
    w = weights(n + k, n, k)
    packed, scales = w4.mx_pack_weights(dev(w))
    ref_c, ref_s = mx.mx_quantize(w, "e2m1")
    assert np.array_equal(host(scales), ref_s.T)
    p = host(packed)                                          # [K/32][N][16]
    nib = np.stack([p & 0xF, p >> 4], axis=-1).reshape(k // 32, n, 32)
    assert np.array_equal(nib, ref_c.reshape(n, k // 32, 32).transpose(1, 0, 2))


ACC = 2.0 ** -12   # bound of the instruction's accumulation error, per unit of sum |a w|


def assert_close(got, ref, absterm, what):
    excess = np.abs(got.astype(np.float64) - ref) - (ATOL + RTOL * np.abs(ref) + ACC * absterm)
    assert (excess <= 0).all(), f"{what}: {(excess > 0).sum()} outside, max excess {excess.max():.3g}"
    rel = np.abs(got.astype(np.float64) - ref) / np.maximum(absterm, 1e-30)
    assert rel.max() < ACC


# ragged M and N against the workgroup tiles, several K steps; the last shape has enough
# 128 x 128 tiles for the LDS-staged kernel (with a half tile at the end of N)
@pytest.mark.parametrize("m,k,n", [(1, 64, 64), (5, 128, 192), (130, 256, 320), (256, 512, 128), (40, 2048, 2560),
                                   (130, 192, 32832)])
def test_mx_linear(m, k, n):
    x = activations(3 * m + k, m, k)
    w = weights(n + 7 * k, n, k)
    packed, scales = w4.mx_pack_weights(dev(w))
    got = host(w4.mx_linear(dev(x), packed, scales))
    qa, sa = mx.mx_quantize(x, "e4m3")
    qw, sw = mx.mx_quantize(w, "e2m1")
    assert_close(got, mx.mx_linear(x, w), mx.mx_abs_terms(qa, sa, qw, sw), f"M={m} K={k} N={n}")


@pytest.mark.parametrize("k,n", [(2048, 2560), (2048, 16384), (8192, 2048)])
def test_mx_linear_prefill_sampled(k, n):
    """M = 512 at the decoder-layer shapes; 192 seeded columns checked against the oracle."""
    m = 512
    x = activations(11 + k, m, k)
    w = weights(13 + n, n, k)
    packed, scales = w4.mx_pack_weights(dev(w))
    got = host(w4.mx_linear(dev(x), packed, scales))
    cols = np.sort(np.random.default_rng(0).choice(n, 192, replace=False))
    qa, sa = mx.mx_quantize(x, "e4m3")
    qw, sw = mx.mx_quantize(w[cols], "e2m1")
    assert_close(got[:, cols], mx.mx_linear_prequantized(qa, sa, qw, sw), mx.mx_abs_terms(qa, sa, qw, sw),
                 f"K={k} N={n}")


def test_mx_linear_repeat_bit_identical():
    x = activations(5, 64, 1024)
    w = weights(6, 256, 1024)
    packed, scales = w4.mx_pack_weights(dev(w))
    xd = dev(x)
    first = host(w4.mx_linear(xd, packed, scales))
    for _ in range(3):
        assert np.array_equal(host(w4.mx_linear(xd, packed, scales)), first)
