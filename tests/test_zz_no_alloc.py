"""w4a8_linear_noalloc (scratch in a static device array, for callers that cannot allocate)
against w4a8_linear through the C ABI: the same kernels, so the same bits, on consecutive calls
whose shapes shrink and grow (prefill GEMM, split-K GEMM, decode GEMV), and against the oracle;
a call beyond the static scratch is rejected before launching anything."""
import ctypes

import numpy as np
import pytest
import torch

import bit_block_quantized_w4a8_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def noalloc(x, packed, ws, out):
    m, k = x.shape
    n = out.shape[1]
    lib = w4.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    return lib.w4a8_linear_noalloc(x.data_ptr(), packed.data_ptr(), ws.data_ptr(), m, k, n, out.data_ptr(),
                                   stream)


def run_case(seed, m, k, n):
    x, qw, sw = synth.linear_inputs(seed, m, k, n, outliers=True)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    xd = dev(x)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    rc = noalloc(xd, packed, ws, out)
    assert rc == w4.W4A8_OK, w4.load_library().w4a8_last_error()
    got = host(out)
    want = host(w4.linear(xd, packed, ws))
    assert np.array_equal(got, want), f"M={m} K={k} N={n}: differs from w4a8_linear"
    rows = np.unique(np.r_[0, m - 1, np.random.default_rng(seed).integers(0, m, 6)])
    ref = oracle.linear(x[rows], qw, sw)
    excess = np.abs(got[rows].astype(np.float64) - ref) - (1e-3 + 1e-3 * np.abs(ref))
    assert excess.max() <= 0, f"M={m} K={k} N={n}: max excess {excess.max():.3g}"


def test_noalloc_matches_linear_on_consecutive_calls():
    w4.init(0)
    size = ctypes.c_size_t(0)
    assert w4.load_library().w4a8_noalloc_scratch_bytes(ctypes.byref(size)) == w4.W4A8_OK
    shapes = [(512, 2048, 2560),   # prefill GEMM (staging 1.2 MB)
              (8, 8192, 2048),     # smaller: split-K GEMM, tickets in the static scratch
              (1, 2048, 16384),    # decode GEMV (no scratch)
              (512, 8192, 2048),   # larger again (staging 4.7 MB)
              (40, 2048, 2048),    # smaller again
              (12, 2048, 16384)]   # small-batch kernel (no scratch)
    assert w4.auto_path(8, 8192, 2048) == w4.PATH_GEMM and w4.auto_path(1, 2048, 16384) == w4.PATH_GEMV
    assert w4.auto_path(12, 2048, 16384) == w4.PATH_BATCH
    for i, (m, k, n) in enumerate(shapes):
        assert w4.linear_scratch_bytes(m, k, n) <= size.value
        run_case(100 + i, m, k, n)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    w4.init(0)
    size = ctypes.c_size_t(0)
    w4.load_library().w4a8_noalloc_scratch_bytes(ctypes.byref(size))
    m, k, n = 4096, 8192, 64
    assert w4.linear_scratch_bytes(m, k, n) > size.value
    x, qw, sw = synth.linear_inputs(7, m, k, n)
    packed, ws = w4.pack_weights(dev(qw), dev(sw))
    out = torch.full((m, n), 3.0, dtype=torch.float32, device=DEV)
    assert noalloc(dev(x), packed, ws, out) == w4.W4A8_EINVAL
    assert b"static scratch" in w4.load_library().w4a8_last_error()
    assert bool((host(out) == 3.0).all())
    # the same shape runs through w4a8_linear with reserved library scratch
    w4.reserve_scratch(w4.linear_scratch_bytes(m, k, n))
    rows = [0, 4095]
    got = host(w4.linear(dev(x), packed, ws))[rows]
    ref = oracle.linear(x[rows], qw, sw)
    assert (np.abs(got - ref) - (1e-3 + 1e-3 * np.abs(ref))).max() <= 0
