"""Python binding of the W4A8 block-32 linear library (libw4a8.so, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/w4a8.h.  PyTorch provides device
memory and the current stream; there is no CPU fallback, and every function
raises if the library is not built or a call fails.

Stage-aware layout of the layer (ML Drift explainer on tech.dede.sh, section
"Stage-aware optimization for large language models"): `linear` runs the
decode GEMV (activations quantised inside the kernel) for few token rows and
the int8-MFMA prefill GEMM for many.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "PATH_AUTO", "PATH_GEMV", "PATH_GEMM", "PATH_BATCH", "W4A8Error", "library_path", "load_library",
    "declared_functions", "init", "pack_weights", "linear", "linear_argmax",
    "quantize_act", "block_sums", "gemv_max_m", "auto_path", "mx_pack_weights", "mx_quantize_act", "mx_linear", "kv_cache", "decode_attention", "Weights", "residual_norm_cast",
    "decoder_layer_workspace", "decoder_layer", "reserve_scratch", "scratch_capacity", "linear_scratch_bytes",
    "decoder_layer_scratch_bytes", "norm_linear_argmax_scratch_bytes", "mx_linear_scratch_bytes",
    "decode_attention_scratch_bytes", "decoder_layer_workspace_offsets", "layer_kernel", "set_option",
    "get_option", "take_device_errors", "decoder_stack", "decoder_layer_attention", "OPTION_RESIDENT_LAYER", "LAYER_CHAIN", "LAYER_GEMM", "LAYER_GEMV4",
    "LAYER_RESIDENT",
]

PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_BATCH = 0, 1, 2, 3
LAYER_CHAIN, LAYER_GEMM, LAYER_GEMV4, LAYER_RESIDENT = 0, 1, 2, 3
OPTION_RESIDENT_LAYER = 1
W4A8_OK, W4A8_EINVAL, W4A8_EUNSUPPORTED, W4A8_EHIP, W4A8_ENOINIT = 0, -1, -2, -3, -4

_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "w4a8.h")
_lib = None


class _CWeights(ctypes.Structure):
    """C struct w4a8_weights."""
    _fields_ = [("packed_w", ctypes.c_void_p), ("w_scales", ctypes.c_void_p),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


class W4A8Error(RuntimeError):
    def __init__(self, fn: str, code: int, message: str):
        super().__init__(f"{fn} returned {code}: {message}")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, "libw4a8.so")


def declared_functions() -> list[str]:
    """Names of the entry points declared in include/w4a8.h."""
    with open(_HEADER) as f:
        text = f.read()
    return re.findall(r"W4A8_API\s+[\w\s\*]+?\b(w4a8_\w+)\s*\(", text)


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m bit_block_quantized_w4a8_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "w4a8_init": ([i32], i32),
        "w4a8_pack_weights": ([p, p, i64, i64, p, p, p], i32),
        "w4a8_linear": ([p, p, p, i64, i64, i64, p, p], i32),
        "w4a8_linear_path": ([p, p, p, i64, i64, i64, p, i32, p], i32),
        "w4a8_linear_noalloc": ([p, p, p, i64, i64, i64, p, p], i32),
        "w4a8_noalloc_scratch_bytes": ([ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_linear_argmax": ([p, p, p, i64, i64, i64, p, p, p], i32),
        "w4a8_norm_linear_argmax": ([p, ctypes.c_float, p, p, i64, i64, i64, p, p, p], i32),
        "w4a8_quantize_act": ([p, i64, i64, p, p, p], i32),
        "w4a8_block_sums": ([p, p, i64, i64, i64, p, i32, p], i32),
        "w4a8_gemv_max_m": ([], i32),
        "w4a8_auto_path": ([i64, i64, i64], i32),
        "w4a8_mx_pack_weights": ([p, i64, i64, p, p, p], i32),
        "w4a8_mx_quantize_act": ([p, i64, i64, p, p, p], i32),
        "w4a8_mx_linear": ([p, p, p, i64, i64, i64, p, p], i32),
        "w4a8_decode_attention": ([p, p, p, p, p, i64, i64, i64, i64, i64, p, p], i32),
        "w4a8_residual_norm_cast": ([p, p, i64, ctypes.c_float, ctypes.c_float, i64, i64, p, p], i32),
        "w4a8_decoder_layer_workspace": ([i64, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                                          ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_decoder_layer": ([p, i64, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                                ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights), ctypes.c_float,
                                ctypes.c_float, p, ctypes.c_size_t, p], i32),
        "w4a8_last_error": ([], ctypes.c_char_p),
        "w4a8_decoder_layer_workspace_offsets": ([i64, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                                                  ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_reserve_scratch": ([ctypes.c_size_t], i32),
        "w4a8_scratch_capacity": ([ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_linear_scratch_bytes": ([i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_decoder_layer_scratch_bytes": ([i64, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                                              ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_norm_linear_argmax_scratch_bytes": ([i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_mx_linear_scratch_bytes": ([i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_decode_attention_scratch_bytes": ([i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)], i32),
        "w4a8_decoder_stack": ([p, i64, i64, ctypes.POINTER(_CWeights), i64, ctypes.c_float, ctypes.c_float, p,
                                ctypes.c_size_t, p], i32),
        "w4a8_decoder_layer_attention": ([p, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                                          ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights), ctypes.c_float,
                                          ctypes.c_float, p, p, i64, i64, i64, i64, i64, p, ctypes.c_size_t, p], i32),
        "w4a8_layer_kernel": ([i64, i64, ctypes.POINTER(_CWeights), ctypes.POINTER(_CWeights),
                               ctypes.POINTER(i32)], i32),
        "w4a8_set_option": ([i32, i32], i32),
        "w4a8_get_option": ([i32, ctypes.POINTER(i32)], i32),
        "w4a8_take_device_errors": ([ctypes.POINTER(ctypes.c_uint32)], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != W4A8_OK:
        msg = load_library().w4a8_last_error().decode(errors="replace")
        raise W4A8Error(fn, code, msg)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got shape {tuple(t.shape)}")


_initialised: set[int] = set()


def init(device: int | None = None) -> None:
    """Select the device and let the library allocate its scratch (idempotent)."""
    dev = torch.cuda.current_device() if device is None else int(device)
    if dev in _initialised:
        return
    _check("w4a8_init", load_library().w4a8_init(dev))
    torch.cuda.set_device(dev)
    _initialised.add(dev)


def reserve_scratch(nbytes: int, device: int | None = None) -> None:
    """Grow the library's scratch work area on the device to at least nbytes (allocates;
    call it before timing or graph capture, never inside)."""
    init(device)
    _check("w4a8_reserve_scratch", load_library().w4a8_reserve_scratch(int(nbytes)))


def scratch_capacity(device: int | None = None) -> int:
    init(device)
    nbytes = ctypes.c_size_t(0)
    _check("w4a8_scratch_capacity", load_library().w4a8_scratch_capacity(ctypes.byref(nbytes)))
    return int(nbytes.value)


def _size_query(fn: str, *args) -> int:
    nbytes = ctypes.c_size_t(0)
    _check(fn, getattr(load_library(), fn)(*args, ctypes.byref(nbytes)))
    return int(nbytes.value)


def linear_scratch_bytes(m: int, k: int, n: int, path: int = PATH_AUTO) -> int:
    return _size_query("w4a8_linear_scratch_bytes", m, k, n, path)


def decoder_layer_scratch_bytes(m: int, h: int, qkv: "Weights", gate_up: "Weights") -> int:
    return _size_query("w4a8_decoder_layer_scratch_bytes", m, h, ctypes.byref(qkv.c), ctypes.byref(gate_up.c))


def norm_linear_argmax_scratch_bytes(m: int, k: int, n: int) -> int:
    return _size_query("w4a8_norm_linear_argmax_scratch_bytes", m, k, n)


def mx_linear_scratch_bytes(m: int, k: int, n: int) -> int:
    return _size_query("w4a8_mx_linear_scratch_bytes", m, k, n)


def decode_attention_scratch_bytes(n_heads: int, n_kv_heads: int, head_dim: int, length: int) -> int:
    return _size_query("w4a8_decode_attention_scratch_bytes", n_heads, n_kv_heads, head_dim, length)


def _ready(t: torch.Tensor):
    init(t.device.index if t.device.index is not None else torch.cuda.current_device())


def pack_weights(q: torch.Tensor, s: torch.Tensor):
    """int8 weights [N][K] in [-8, 7] + fp16 scales [N][K/32] -> (packed uint8 [K/32][N][16], fp16 [K/32][N])."""
    _need(q, "q", torch.int8, 2)
    _need(s, "s", torch.float16, 2)
    n, k = q.shape
    if s.shape != (n, k // 32):
        raise ValueError(f"scales must be [{n}][{k // 32}], got {tuple(s.shape)}")
    _ready(q)
    packed = torch.empty((k // 32, n, 16), dtype=torch.uint8, device=q.device)
    w_scales = torch.empty((k // 32, n), dtype=torch.float16, device=q.device)
    _check("w4a8_pack_weights", load_library().w4a8_pack_weights(
        q.data_ptr(), s.data_ptr(), k, n, packed.data_ptr(), w_scales.data_ptr(), _stream(q)))
    return packed, w_scales


def _weights_shape(packed: torch.Tensor, w_scales: torch.Tensor):
    _need(packed, "packed_w", torch.uint8, 3)
    _need(w_scales, "w_scales", torch.float16, 2)
    nb, n, width = packed.shape
    if width != 16 or w_scales.shape != (nb, n):
        raise ValueError("packed_w must be [K/32][N][16] and w_scales [K/32][N]")
    return nb * 32, n


def linear(x: torch.Tensor, packed: torch.Tensor, w_scales: torch.Tensor, path: int = PATH_AUTO,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """fp16 activations [M][K] -> fp32 [M][N] through the W4A8 block-32 linear layer."""
    _need(x, "x", torch.float16, 2)
    k, n = _weights_shape(packed, w_scales)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has K = {x.shape[1]}, weights have K = {k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    else:
        _need(out, "out", torch.float32, 2)
        if out.shape != (m, n):
            raise ValueError("out has the wrong shape")
    _ready(x)
    _check("w4a8_linear_path", load_library().w4a8_linear_path(
        x.data_ptr(), packed.data_ptr(), w_scales.data_ptr(), m, k, n, out.data_ptr(), path,
        _stream(x)))
    return out


def linear_argmax(x: torch.Tensor, packed: torch.Tensor, w_scales: torch.Tensor,
                  logits: torch.Tensor | bool | None = None, argmax: torch.Tensor | None = None):
    """Linear layer + fused argmax per row.  Returns argmax int32 [M], or (argmax, logits)
    when `logits` is True or a preallocated fp32 [M][N] tensor."""
    _need(x, "x", torch.float16, 2)
    k, n = _weights_shape(packed, w_scales)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has K = {x.shape[1]}, weights have K = {k}")
    want_logits = logits is not None and logits is not False
    if logits is True:
        logits = torch.empty((m, n), dtype=torch.float32, device=x.device)
    elif want_logits:
        _need(logits, "logits", torch.float32, 2)
    if argmax is None:
        argmax = torch.empty((m,), dtype=torch.int32, device=x.device)
    else:
        _need(argmax, "argmax", torch.int32, 1)
    _ready(x)
    _check("w4a8_linear_argmax", load_library().w4a8_linear_argmax(
        x.data_ptr(), packed.data_ptr(), w_scales.data_ptr(), m, k, n,
        logits.data_ptr() if want_logits else None, argmax.data_ptr(), _stream(x)))
    return (argmax, logits) if want_logits else argmax


def norm_linear_argmax(x: torch.Tensor, packed: torch.Tensor, w_scales: torch.Tensor, eps: float = 1e-6,
                       logits: torch.Tensor | bool | None = None, argmax: torch.Tensor | None = None):
    """LM-head argmax on the fp32 residual stream: argmax of linear(fp16(x / rms(x))) per row.
    Returns argmax int32 [M], or (argmax, logits) as linear_argmax does."""
    _need(x, "x", torch.float32, 2)
    k, n = _weights_shape(packed, w_scales)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x has K = {x.shape[1]}, weights have K = {k}")
    want_logits = logits is not None and logits is not False
    if logits is True:
        logits = torch.empty((m, n), dtype=torch.float32, device=x.device)
    elif want_logits:
        _need(logits, "logits", torch.float32, 2)
    if argmax is None:
        argmax = torch.empty((m,), dtype=torch.int32, device=x.device)
    else:
        _need(argmax, "argmax", torch.int32, 1)
    _ready(x)
    _check("w4a8_norm_linear_argmax", load_library().w4a8_norm_linear_argmax(
        x.data_ptr(), eps, packed.data_ptr(), w_scales.data_ptr(), m, k, n,
        logits.data_ptr() if want_logits else None, argmax.data_ptr(), _stream(x)))
    return (argmax, logits) if want_logits else argmax


def quantize_act(x: torch.Tensor):
    """The in-kernel activation quantiser on its own: (qx int8 [M][K], sx fp32 [M][K/32])."""
    _need(x, "x", torch.float16, 2)
    m, k = x.shape
    qx = torch.empty((m, k), dtype=torch.int8, device=x.device)
    sx = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _ready(x)
    _check("w4a8_quantize_act", load_library().w4a8_quantize_act(
        x.data_ptr(), m, k, qx.data_ptr(), sx.data_ptr(), _stream(x)))
    return qx, sx


def block_sums(x: torch.Tensor, packed: torch.Tensor, path: int = PATH_AUTO) -> torch.Tensor:
    """Unscaled integer block sums int32 [M][N][K/32] as the chosen kernel forms them."""
    _need(x, "x", torch.float16, 2)
    _need(packed, "packed_w", torch.uint8, 3)
    nb, n, _ = packed.shape
    m, k = x.shape
    if k != nb * 32:
        raise ValueError("x and packed_w disagree on K")
    sums = torch.empty((m, n, nb), dtype=torch.int32, device=x.device)
    _ready(x)
    _check("w4a8_block_sums", load_library().w4a8_block_sums(
        x.data_ptr(), packed.data_ptr(), m, k, n, sums.data_ptr(), path, _stream(x)))
    return sums


def gemv_max_m() -> int:
    return int(load_library().w4a8_gemv_max_m())


def mx_pack_weights(w: torch.Tensor):
    """MXFP4 weights from fp16 w [N][K]: (packed uint8 [K/32][N][16], scales uint8 [K/32][N])."""
    _need(w, "w", torch.float16, 2)
    n, k = w.shape
    packed = torch.empty((k // 32, n, 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty((k // 32, n), dtype=torch.uint8, device=w.device)
    _ready(w)
    _check("w4a8_mx_pack_weights", load_library().w4a8_mx_pack_weights(
        w.data_ptr(), k, n, packed.data_ptr(), scales.data_ptr(), _stream(w)))
    return packed, scales


def mx_quantize_act(x: torch.Tensor):
    """MXFP8 activations from fp16 x [M][K]: (codes uint8 [K/32][M][32], scales uint8 [K/32][M])."""
    _need(x, "x", torch.float16, 2)
    m, k = x.shape
    codes = torch.empty((k // 32, m, 32), dtype=torch.uint8, device=x.device)
    scales = torch.empty((k // 32, m), dtype=torch.uint8, device=x.device)
    _ready(x)
    _check("w4a8_mx_quantize_act", load_library().w4a8_mx_quantize_act(
        x.data_ptr(), m, k, codes.data_ptr(), scales.data_ptr(), _stream(x)))
    return codes, scales


def mx_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None):
    """fp32 [M][N] = MXFP8(x) . MXFP4(W)^T (see w4a8_mx_linear)."""
    _need(x, "x", torch.float16, 2)
    _need(packed, "packed", torch.uint8, 3)
    _need(scales, "scales", torch.uint8, 2)
    m, k = x.shape
    n = packed.shape[1]
    if packed.shape != (k // 32, n, 16) or scales.shape != (k // 32, n):
        raise ValueError(f"MX weights of shape {tuple(packed.shape)} / {tuple(scales.shape)} do not match K = {k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _ready(x)
    _check("w4a8_mx_linear", load_library().w4a8_mx_linear(
        x.data_ptr(), packed.data_ptr(), scales.data_ptr(), m, k, n, out.data_ptr(), _stream(x)))
    return out


def kv_cache(n_kv_heads: int, head_dim: int, capacity: int, device=None):
    """Zeroed fp16 (k_cache [n_kv_heads][capacity][head_dim], v_cache [n_kv_heads][head_dim][capacity])
    in the storage order w4a8_decode_attention reads."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return (torch.zeros((n_kv_heads, capacity, head_dim), dtype=torch.float16, device=dev),
            torch.zeros((n_kv_heads, head_dim, capacity), dtype=torch.float16, device=dev))


def decode_attention(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, length: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp16 [Hq][D] attention of the newest token (position length - 1, whose key and value
    this call writes into the caches) over positions 0 .. length - 1 (see w4a8_decode_attention)."""
    _need(q, "q", torch.float32, 2)
    _need(k_new, "k_new", torch.float32, 2)
    _need(v_new, "v_new", torch.float32, 2)
    _need(k_cache, "k_cache", torch.float16, 3)
    _need(v_cache, "v_cache", torch.float16, 3)
    hq, d = q.shape
    hkv, cap = k_new.shape[0], k_cache.shape[1]
    if k_new.shape != (hkv, d) or v_new.shape != (hkv, d):
        raise ValueError(f"k_new / v_new must be [{hkv}][{d}]")
    if k_cache.shape != (hkv, cap, d) or v_cache.shape != (hkv, d, cap):
        raise ValueError(f"caches of shape {tuple(k_cache.shape)} / {tuple(v_cache.shape)} do not match "
                         f"[{hkv}][capacity][{d}] / [{hkv}][{d}][capacity]")
    if out is None:
        out = torch.empty((hq, d), dtype=torch.float16, device=q.device)
    _ready(q)
    _check("w4a8_decode_attention", load_library().w4a8_decode_attention(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        hq, hkv, d, length, cap, out.data_ptr(), _stream(q)))
    return out


def auto_path(m: int, k: int, n: int) -> int:
    """PATH_GEMV, PATH_GEMM or PATH_BATCH: the kernel PATH_AUTO runs for an m x k by k x n linear."""
    return int(load_library().w4a8_auto_path(m, k, n))


class Weights:
    """A packed weight matrix (device tensors) and its C descriptor."""

    def __init__(self, packed: torch.Tensor, w_scales: torch.Tensor):
        k, n = _weights_shape(packed, w_scales)
        self.packed, self.w_scales, self.K, self.N = packed, w_scales, k, n
        self.c = _CWeights(packed.data_ptr(), w_scales.data_ptr(), k, n)

    @classmethod
    def pack(cls, q: torch.Tensor, s: torch.Tensor) -> "Weights":
        return cls(*pack_weights(q, s))


def residual_norm_cast(x: torch.Tensor, d: torch.Tensor | None = None, alpha: float = 0.0,
                       eps: float = 1e-6, y: torch.Tensor | None = None, want_y: bool = True):
    """x (fp32 [M][H], in place) += alpha * d[:, :H] if d is given; returns fp16(x / rms(x)) or None."""
    _need(x, "x", torch.float32, 2)
    m, h = x.shape
    ld = 0
    if d is not None:
        _need(d, "d", torch.float32, 2)
        if d.shape[0] != m or d.shape[1] < h:
            raise ValueError("d must be [M][>= H]")
        ld = d.shape[1]
    if want_y and y is None:
        y = torch.empty((m, h), dtype=torch.float16, device=x.device)
    elif y is not None:
        _need(y, "y", torch.float16, 2)
    _ready(x)
    _check("w4a8_residual_norm_cast", load_library().w4a8_residual_norm_cast(
        x.data_ptr(), d.data_ptr() if d is not None else None, ld, alpha, eps, m, h,
        y.data_ptr() if want_y else None, _stream(x)))
    return y if want_y else None


def decoder_layer_workspace(m: int, h: int, qkv: Weights, gate_up: Weights) -> int:
    nbytes = ctypes.c_size_t(0)
    _check("w4a8_decoder_layer_workspace", load_library().w4a8_decoder_layer_workspace(
        m, h, ctypes.byref(qkv.c), ctypes.byref(gate_up.c), ctypes.byref(nbytes)))
    return int(nbytes.value)


def decoder_layer_workspace_offsets(m: int, h: int, qkv: Weights, gate_up: Weights) -> dict:
    """Byte offsets of the intermediates q, a, o, n, g, u, d in the layer workspace."""
    offs = (ctypes.c_size_t * 7)()
    _check("w4a8_decoder_layer_workspace_offsets", load_library().w4a8_decoder_layer_workspace_offsets(
        m, h, ctypes.byref(qkv.c), ctypes.byref(gate_up.c), offs))
    return dict(zip("q a o n g u d".split(), (int(v) for v in offs)))


def layer_kernel(m: int, h: int, qkv: Weights, gate_up: Weights) -> int:
    """LAYER_CHAIN, LAYER_GEMM, LAYER_GEMV4 or LAYER_RESIDENT: how decoder_layer runs this shape here."""
    k = ctypes.c_int(0)
    _check("w4a8_layer_kernel", load_library().w4a8_layer_kernel(
        m, h, ctypes.byref(qkv.c), ctypes.byref(gate_up.c), ctypes.byref(k)))
    return int(k.value)


def set_option(option: int, value: int) -> None:
    _check("w4a8_set_option", load_library().w4a8_set_option(option, value))


def get_option(option: int) -> int:
    v = ctypes.c_int(0)
    _check("w4a8_get_option", load_library().w4a8_get_option(option, ctypes.byref(v)))
    return int(v.value)


def take_device_errors() -> int:
    """Error word of the current device's kernels since the last call (0: none), then cleared."""
    v = ctypes.c_uint32(0)
    _check("w4a8_take_device_errors", load_library().w4a8_take_device_errors(ctypes.byref(v)))
    return int(v.value)


def decoder_layer(x: torch.Tensor, qkv: Weights, o: Weights, gate_up: Weights, down: Weights,
                  residual_scale: float, eps: float, workspace: torch.Tensor) -> torch.Tensor:
    """One synthetic decoder layer in place on the fp32 residual stream x [M][H]."""
    _need(x, "x", torch.float32, 2)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    m, h = x.shape
    _ready(x)
    _check("w4a8_decoder_layer", load_library().w4a8_decoder_layer(
        x.data_ptr(), m, h, ctypes.byref(qkv.c), ctypes.byref(o.c), ctypes.byref(gate_up.c),
        ctypes.byref(down.c), residual_scale, eps, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(x)))
    return x


def decoder_stack(x: torch.Tensor, layers: list, residual_scale: float, eps: float,
                  workspace: torch.Tensor) -> torch.Tensor:
    """Decoder layers in order, in place on the fp32 residual stream x [M][H].

    layers: a list of dicts with Weights under "qkv", "o", "gate_up" and "down".
    """
    _need(x, "x", torch.float32, 2)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    if not layers:
        raise ValueError("layers must not be empty")
    table = (_CWeights * (4 * len(layers)))()
    for i, lw in enumerate(layers):
        for j, name in enumerate(("qkv", "o", "gate_up", "down")):
            table[4 * i + j] = lw[name].c
    m, h = x.shape
    _ready(x)
    _check("w4a8_decoder_stack", load_library().w4a8_decoder_stack(
        x.data_ptr(), m, h, table, len(layers), residual_scale, eps, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(x)))
    return x


def decoder_layer_attention(x: torch.Tensor, qkv: Weights, o: Weights, gate_up: Weights, down: Weights,
                            residual_scale: float, eps: float, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            n_heads: int, length: int, workspace: torch.Tensor) -> torch.Tensor:
    """One decode token through a decoder layer with attention between qkv and o, in place on x [1][H]."""
    _need(x, "x", torch.float32, 2)
    _need(k_cache, "k_cache", torch.float16, 3)
    _need(v_cache, "v_cache", torch.float16, 3)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    m, h = x.shape
    if m != 1:
        raise ValueError("decoder_layer_attention takes one token row")
    hkv, cap, d = k_cache.shape
    if v_cache.shape != (hkv, d, cap):
        raise ValueError(f"v_cache must be [{hkv}][{d}][{cap}]")
    _ready(x)
    _check("w4a8_decoder_layer_attention", load_library().w4a8_decoder_layer_attention(
        x.data_ptr(), h, ctypes.byref(qkv.c), ctypes.byref(o.c), ctypes.byref(gate_up.c), ctypes.byref(down.c),
        residual_scale, eps, k_cache.data_ptr(), v_cache.data_ptr(), n_heads, hkv, d, length, cap,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(x)))
    return x
