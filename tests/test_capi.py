"""The C ABI library on a machine without a GPU: it loads, exports every declared
entry point, and rejects invalid arguments before touching the device."""
import ctypes

import pytest

import bit_block_quantized_w4a8_amd as w4


@pytest.fixture(scope="module")
def lib():
    return w4.load_library()


def test_exports_every_declared_symbol(lib):
    names = w4.declared_functions()
    assert len(names) == 34, names
    for name in names:
        assert hasattr(lib, name), name


def test_gemv_threshold(lib):
    assert 1 <= lib.w4a8_gemv_max_m() <= 64


def test_auto_path_rule():
    """Host-side stage rule: GEMV at M = 1, at M = 2 too where the small-batch kernel does not
    run, and through M = 4 for weight matrices of at most 2^25 values; then the small-batch kernel
    through M = 16 where it runs and either N >= 8192 or K <= 4096; the GEMM above (the
    environment override is not set under pytest)."""
    gemv, gemm, batch = w4.PATH_GEMV, w4.PATH_GEMM, w4.PATH_BATCH
    for k, n in [(2048, 2560), (2048, 16384)]:
        assert [w4.auto_path(m, k, n) for m in (1, 2, 3, 4, 5, 16, 17, 512)] == [gemv] * 4 + [batch] * 2 + [gemm] * 2
    assert [w4.auto_path(m, 8192, 2048) for m in (1, 4, 5, 16, 512)] == [gemv, gemv, gemm, gemm, gemm]
    assert [w4.auto_path(m, 4096, 14336) for m in (1, 2, 3, 4, 8, 16, 17)] == [gemv] + [batch] * 5 + [gemm]
    # outside the small-batch kernel's shapes (K not a multiple of 256) the GEMM takes over
    assert [w4.auto_path(m, 4128, 14336) for m in (2, 3, 16)] == [gemv, gemm, gemm]


ALIGNED = 1 << 20       # fake, suitably aligned device addresses: never dereferenced
P = ctypes.c_void_p


def _linear(lib, x=ALIGNED, pw=ALIGNED, ws=ALIGNED, m=1, k=64, n=128, out=ALIGNED, path=0):
    return lib.w4a8_linear_path(P(x), P(pw), P(ws), m, k, n, P(out), path, None)


@pytest.mark.parametrize("kw", [
    dict(x=0), dict(pw=0), dict(ws=0), dict(out=0),
    dict(m=0), dict(m=-3), dict(k=0), dict(k=48), dict(k=16), dict(n=0), dict(n=96), dict(n=32),
    dict(x=ALIGNED + 2), dict(x=ALIGNED + 8), dict(pw=ALIGNED + 8), dict(ws=ALIGNED + 2), dict(ws=ALIGNED + 8),
    dict(out=ALIGNED + 4),
    dict(path=4), dict(path=-1), dict(path=3, m=17, k=256), dict(path=3, k=288), dict(path=3, k=64),
])
def test_linear_rejects_bad_arguments(lib, kw):
    assert _linear(lib, **kw) == w4.W4A8_EINVAL
    assert lib.w4a8_last_error()


def test_valid_arguments_need_init(lib):
    assert _linear(lib) == w4.W4A8_ENOINIT
    assert _linear(lib, m=16, k=256, path=w4.PATH_BATCH) == w4.W4A8_ENOINIT
    assert b"w4a8_init" in lib.w4a8_last_error()


def test_other_entry_points_validate(lib):
    assert lib.w4a8_linear(P(0), P(ALIGNED), P(ALIGNED), 1, 64, 128, P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_linear_argmax(P(ALIGNED), P(ALIGNED), P(ALIGNED), 65, 64, 128, P(0), P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_linear_argmax(P(ALIGNED), P(ALIGNED), P(ALIGNED), 1, 64, 128, P(0), P(0), None) == w4.W4A8_EINVAL
    assert lib.w4a8_linear_argmax(P(ALIGNED), P(ALIGNED), P(ALIGNED), 1, 64, 128, P(ALIGNED + 4), P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_linear_argmax(P(ALIGNED), P(ALIGNED), P(ALIGNED), 1, 64, 128, P(0), P(ALIGNED), None) == w4.W4A8_ENOINIT
    assert lib.w4a8_quantize_act(P(ALIGNED), 2, 40, P(ALIGNED), P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_quantize_act(P(ALIGNED), 2, 64, P(0), P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_block_sums(P(ALIGNED), P(ALIGNED), 1, 64, 128, P(ALIGNED + 4), 0, None) == w4.W4A8_EINVAL
    assert lib.w4a8_block_sums(P(ALIGNED), P(ALIGNED), 1, 64, 128, P(ALIGNED), 7, None) == w4.W4A8_EINVAL
    assert lib.w4a8_pack_weights(P(ALIGNED), P(ALIGNED), 64, 100, P(ALIGNED), P(ALIGNED), None) == w4.W4A8_EINVAL
    assert lib.w4a8_pack_weights(P(ALIGNED), P(ALIGNED), 64, 128, P(ALIGNED + 1), P(ALIGNED), None) == w4.W4A8_EINVAL


def test_norm_linear_argmax_validates(lib):
    f = ctypes.c_float
    ok = dict(x=ALIGNED, eps=1e-6, pw=ALIGNED, ws=ALIGNED, m=1, k=64, n=128, logits=0, am=ALIGNED)

    def call(**kw):
        a = {**ok, **kw}
        return lib.w4a8_norm_linear_argmax(P(a["x"]), f(a["eps"]), P(a["pw"]), P(a["ws"]), a["m"], a["k"], a["n"],
                                           P(a["logits"]), P(a["am"]), None)
    for bad in [dict(x=0), dict(x=ALIGNED + 8), dict(eps=-1.0), dict(m=65), dict(k=48), dict(n=96),
                dict(am=0), dict(am=ALIGNED + 2), dict(logits=ALIGNED + 4), dict(pw=ALIGNED + 8)]:
        assert call(**bad) == w4.W4A8_EINVAL, bad
    assert call() == w4.W4A8_ENOINIT


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        w4.linear(torch.zeros(1, 32, dtype=torch.float16), torch.zeros(1, 64, 16, dtype=torch.uint8),
                  torch.zeros(1, 64, dtype=torch.float16))


def test_mx_entry_points_validate(lib):
    """MX entry points reject null pointers, K not a multiple of 64, N not a multiple of 64
    and misaligned operands before any HIP call; valid arguments then need w4a8_init."""
    A = ALIGNED
    assert lib.w4a8_mx_linear(P(A), P(A), P(A), 4, 96, 128, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(A), P(A), P(A), 4, 128, 96, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(0), P(A), P(A), 4, 128, 128, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(A), P(A), P(0), 4, 128, 128, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(A + 8), P(A), P(A), 4, 128, 128, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(A), P(A), P(A), 0, 128, 128, P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear(P(A), P(A), P(A), 4, 128, 128, P(A), None) == w4.W4A8_ENOINIT
    assert lib.w4a8_mx_pack_weights(P(A), 32, 128, P(A), P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_pack_weights(P(A), 64, 128, P(A + 4), P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_pack_weights(P(A), 64, 128, P(A), P(A), None) == w4.W4A8_ENOINIT
    assert lib.w4a8_mx_quantize_act(P(A), 3, 96, P(A), P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_quantize_act(P(A), 3, 128, P(A + 4), P(A), None) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_quantize_act(P(A), 3, 128, P(A), P(A), None) == w4.W4A8_ENOINIT


def test_decode_attention_validates(lib):
    """w4a8_decode_attention rejects null or misaligned pointers, unsupported head sizes,
    group sizes above 8, a capacity that is not a multiple of 64 and a length outside
    [1, capacity] before any HIP call; valid arguments then need w4a8_init."""
    A = ALIGNED
    f = lib.w4a8_decode_attention

    def call(q=A, kn=A, vn=A, kc=A, vc=A, hq=8, hkv=1, d=256, length=640, cap=640, out=A):
        return f(P(q), P(kn), P(vn), P(kc), P(vc), hq, hkv, d, length, cap, P(out), None)

    assert call(q=0) == w4.W4A8_EINVAL
    assert call(vc=0) == w4.W4A8_EINVAL
    assert call(out=A + 8) == w4.W4A8_EINVAL
    assert call(kc=A + 2) == w4.W4A8_EINVAL
    assert call(d=96) == w4.W4A8_EINVAL
    assert call(hq=9, hkv=1) == w4.W4A8_EINVAL
    assert call(hq=6, hkv=4) == w4.W4A8_EINVAL
    assert call(hkv=0) == w4.W4A8_EINVAL
    assert call(cap=600, length=600) == w4.W4A8_EINVAL
    assert call(length=0) == w4.W4A8_EINVAL
    assert call(length=641) == w4.W4A8_EINVAL
    assert call() == w4.W4A8_ENOINIT
    assert call(hq=16, hkv=2, d=64, length=1, cap=64) == w4.W4A8_ENOINIT


def test_scratch_sizes_on_the_host(lib):
    """The sizing queries need no device: the decode GEMV needs no scratch, the prefill
    GEMM its staging (codes and fp32 scales of every 32-row padded block, 256-byte aligned)."""
    assert w4.linear_scratch_bytes(1, 2048, 16384, w4.PATH_GEMV) == 0
    assert w4.linear_scratch_bytes(1, 2048, 16384) == 0
    nb, m_pad = 2048 // 32, 512
    assert w4.linear_scratch_bytes(512, 2048, 16384) == nb * m_pad * 32 + nb * m_pad * 4
    assert w4.linear_scratch_bytes(512, 2048, 16384, w4.PATH_GEMM) == nb * m_pad * 32 + nb * m_pad * 4
    assert w4.linear_scratch_bytes(16, 4096, 14336, w4.PATH_BATCH) == 0
    assert w4.norm_linear_argmax_scratch_bytes(1, 2048, 262144) == 0
    assert w4.norm_linear_argmax_scratch_bytes(2, 256, 4096) == 2 * 256 * 2
    assert w4.mx_linear_scratch_bytes(512, 2048, 2560) == 512 * 2048 + 512 * 64
    assert w4.decode_attention_scratch_bytes(8, 1, 256, 640) > 0


@pytest.mark.parametrize("args", [(0, 64, 64, 0), (1, 48, 64, 0), (1, 64, 96, 0), (1, 64, 64, 7),
                                  (17, 256, 64, 3), (1, 288, 64, 3)])
def test_scratch_queries_reject_bad_shapes(lib, args):
    n = ctypes.c_size_t(0)
    assert lib.w4a8_linear_scratch_bytes(*args, ctypes.byref(n)) == w4.W4A8_EINVAL
    n = ctypes.c_size_t(0)
    assert lib.w4a8_decode_attention_scratch_bytes(8, 3, 256, 640, ctypes.byref(n)) == w4.W4A8_EINVAL
    assert lib.w4a8_decode_attention_scratch_bytes(8, 1, 96, 640, ctypes.byref(n)) == w4.W4A8_EINVAL
    assert lib.w4a8_mx_linear_scratch_bytes(1, 96, 64, ctypes.byref(n)) == w4.W4A8_EINVAL


def test_reserve_needs_init(lib):
    assert lib.w4a8_reserve_scratch(1 << 20) == w4.W4A8_ENOINIT
    n = ctypes.c_size_t(0)
    assert lib.w4a8_scratch_capacity(ctypes.byref(n)) == w4.W4A8_ENOINIT


def test_options_on_the_host(lib):
    """The resident-layer option takes 0 or 1 and needs no device; unknown options and values are rejected."""
    assert w4.get_option(w4.OPTION_RESIDENT_LAYER) == 1
    try:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 0)
        assert w4.get_option(w4.OPTION_RESIDENT_LAYER) == 0
    finally:
        w4.set_option(w4.OPTION_RESIDENT_LAYER, 1)
    assert lib.w4a8_set_option(w4.OPTION_RESIDENT_LAYER, 2) == w4.W4A8_EINVAL
    assert lib.w4a8_set_option(99, 0) == w4.W4A8_EINVAL
    v = ctypes.c_int(0)
    assert lib.w4a8_get_option(99, ctypes.byref(v)) == w4.W4A8_EINVAL
    assert lib.w4a8_get_option(w4.OPTION_RESIDENT_LAYER, None) == w4.W4A8_EINVAL


def test_device_queries_need_init(lib):
    e = ctypes.c_uint32(0)
    assert lib.w4a8_take_device_errors(ctypes.byref(e)) == w4.W4A8_ENOINIT
    assert lib.w4a8_take_device_errors(None) == w4.W4A8_EINVAL
    qkv = w4._CWeights(ALIGNED, ALIGNED, 2048, 2560)
    gu = w4._CWeights(ALIGNED, ALIGNED, 2048, 16384)
    k = ctypes.c_int(-1)
    assert lib.w4a8_layer_kernel(1, 2048, ctypes.byref(qkv), ctypes.byref(gu), ctypes.byref(k)) == w4.W4A8_ENOINIT
    assert lib.w4a8_layer_kernel(1, 2048, ctypes.byref(qkv), ctypes.byref(gu), None) == w4.W4A8_EINVAL
    bad = w4._CWeights(ALIGNED, ALIGNED, 2048, 100)
    assert lib.w4a8_layer_kernel(1, 2048, ctypes.byref(qkv), ctypes.byref(bad), ctypes.byref(k)) == w4.W4A8_EINVAL


def test_decoder_stack_validates(lib):
    """Argument errors come before the device is needed (EINVAL), a valid call without init is ENOINIT."""
    def table(n, gu_n=16384):
        t = (w4._CWeights * (4 * n))()
        for i in range(n):
            t[4 * i + 0] = w4._CWeights(ALIGNED, ALIGNED, 2048, 2560)
            t[4 * i + 1] = w4._CWeights(ALIGNED, ALIGNED, 2048, 2048)
            t[4 * i + 2] = w4._CWeights(ALIGNED, ALIGNED, 2048, gu_n)
            t[4 * i + 3] = w4._CWeights(ALIGNED, ALIGNED, gu_n // 2, 2048)
        return t

    def call(t, n, x=ALIGNED, ws=ALIGNED, nbytes=1 << 30):
        return lib.w4a8_decoder_stack(P(x), 1, 2048, t, n, ctypes.c_float(0.01), ctypes.c_float(1e-6), P(ws),
                                      nbytes, None)

    t = table(3)
    assert call(t, 3) == w4.W4A8_ENOINIT
    assert call(t, 0) == w4.W4A8_EINVAL
    assert call(None, 3) == w4.W4A8_EINVAL
    assert call(t, 3, x=ALIGNED + 4) == w4.W4A8_EINVAL
    assert call(t, 3, ws=ALIGNED + 16) == w4.W4A8_EINVAL
    assert call(t, 3, nbytes=64) == w4.W4A8_EINVAL
    t[4 * 2 + 2] = w4._CWeights(ALIGNED, ALIGNED, 2048, 8192)   # layer 2's gate_up differs from layer 0's
    t[4 * 2 + 3] = w4._CWeights(ALIGNED, ALIGNED, 4096, 2048)
    assert call(t, 3) == w4.W4A8_EINVAL
    t = table(2)
    t[4 * 1 + 1] = w4._CWeights(ALIGNED, ALIGNED, 2048, 1024)   # o not H x H
    assert call(t, 2) == w4.W4A8_EINVAL


def test_decoder_layer_attention_validates(lib):
    """Shape rules of the layer with attention: H = n_heads * head_dim, qkv.N = (n_heads + 2 n_kv_heads)
    * head_dim, length <= capacity; a valid call without init is ENOINIT."""
    def cw(k, n):
        return ctypes.byref(w4._CWeights(ALIGNED, ALIGNED, k, n))

    def call(h=2048, nq=2560, hq=8, hkv=1, d=256, length=513, cap=640, ws=1 << 30):
        return lib.w4a8_decoder_layer_attention(P(ALIGNED), h, cw(h, nq), cw(h, h), cw(h, 16384), cw(8192, h),
                                                ctypes.c_float(0.01), ctypes.c_float(1e-6), P(ALIGNED), P(ALIGNED),
                                                hq, hkv, d, length, cap, P(ALIGNED), ws, None)

    assert call() == w4.W4A8_ENOINIT
    assert call(hq=4) == w4.W4A8_EINVAL            # 4 x 256 != 2048
    assert call(nq=2304) == w4.W4A8_EINVAL         # no room for the value head
    assert call(length=641) == w4.W4A8_EINVAL
    assert call(cap=600) == w4.W4A8_EINVAL
    assert call(d=96) == w4.W4A8_EINVAL
    assert call(ws=64) == w4.W4A8_EINVAL
