"""ctypes binding of the plain C reference oracle/w4a8_ref.c -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may use it.  It computes the same scheme as oracle/__init__.py (quantise,
exact integer block dots, fp64 scaled sum over blocks in ascending order), in
plain C with OpenMP over output columns; tests/test_oracle_cref.py holds it to
the numpy oracle bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "w4a8_ref.c")
LIB = os.path.join(HERE, "libw4a8_ref.so")
_lib = None


def build() -> str:
    """Compile w4a8_ref.c with the host C compiler (IEEE arithmetic, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-o", LIB + ".tmp", SOURCE, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.w4a8_ref_quantize.argtypes = [p, i64, i64, p, p]
        lib.w4a8_ref_block_sums.argtypes = [p, p, i64, i64, i64, p, i32]
        lib.w4a8_ref_scaled.argtypes = [p, p, p, p, i64, i64, i64, p, i32]
        lib.w4a8_ref_linear.argtypes = [p, p, p, i64, i64, i64, p, p, p, i32]
        lib.w4a8_ref_max_threads.restype = i32
        for f in ("w4a8_ref_quantize", "w4a8_ref_block_sums", "w4a8_ref_scaled", "w4a8_ref_linear"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize(x16: np.ndarray):
    x = np.ascontiguousarray(x16, dtype=np.float16)
    m, k = x.shape
    qx = np.empty((m, k), np.int8)
    sx = np.empty((m, k // 32), np.float32)
    load().w4a8_ref_quantize(_ptr(x.view(np.uint16)), m, k, _ptr(qx), _ptr(sx))
    return qx, sx


def block_sums(qx: np.ndarray, qw: np.ndarray, threads: int = 1) -> np.ndarray:
    a = np.ascontiguousarray(qx, np.int8)
    w = np.ascontiguousarray(qw, np.int8)
    m, k = a.shape
    n = w.shape[0]
    out = np.empty((m, n, k // 32), np.int32)
    load().w4a8_ref_block_sums(_ptr(a), _ptr(w), m, k, n, _ptr(out), threads)
    return out


def scaled(qx, sx, qw, sw16, threads: int = 1) -> np.ndarray:
    a = np.ascontiguousarray(qx, np.int8)
    s = np.ascontiguousarray(sx, np.float32)
    w = np.ascontiguousarray(qw, np.int8)
    sw = np.ascontiguousarray(sw16, np.float16)
    m, k = a.shape
    n = w.shape[0]
    out = np.empty((m, n), np.float64)
    load().w4a8_ref_scaled(_ptr(a), _ptr(s), _ptr(w), _ptr(sw.view(np.uint16)), m, k, n, _ptr(out), threads)
    return out


def linear(x16, qw, sw16, threads: int = 1) -> np.ndarray:
    """fp64 [M][N] output of the W4A8 block-32 linear (see oracle/w4a8_ref.c)."""
    x = np.ascontiguousarray(x16, np.float16)
    w = np.ascontiguousarray(qw, np.int8)
    sw = np.ascontiguousarray(sw16, np.float16)
    m, k = x.shape
    n = w.shape[0]
    qx = np.empty((m, k), np.int8)
    sx = np.empty((m, k // 32), np.float32)
    out = np.empty((m, n), np.float64)
    load().w4a8_ref_linear(_ptr(x.view(np.uint16)), _ptr(w), _ptr(sw.view(np.uint16)), m, k, n, _ptr(qx), _ptr(sx),
                           _ptr(out), threads)
    return out


def max_threads() -> int:
    return int(load().w4a8_ref_max_threads())
