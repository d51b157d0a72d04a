"""CPU oracle for the MX variant of the block-32 linear -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark may import this
module; the GPU library shares no code with it.

The pages fix 4-bit weights in blocks of 32 (ML Drift explainer on
tech.dede.sh, section "Stage-aware optimization for large language models").
This variant keeps the 4 bits and the block of 32 but takes its number
formats from the OCP Microscaling (MX) v1.0 specification, whose scaled
formats gfx950's block-scaled matrix instructions consume:

  * a block of 32 values shares one E8M0 scale X = 2^(c - 127), c in 0..254;
  * weights are FP4 E2M1 elements (MXFP4), activations FP8 E4M3 elements
    (MXFP8); a value is element * X;
  * conversion of a block (the specification's float-to-MX steps):
      shared_exp = floor(log2(max |V_i|)) - emax_elem
        (emax_elem = 8 for E4M3, whose largest normal is 1.75 * 2^8 = 448;
         2 for E2M1, whose largest normal is 1.5 * 2^2 = 6)
      X = 2^shared_exp
      P_i = V_i / X rounded to the element format, nearest with ties to
            even, and clamped to the largest normal (V_i / X can reach
            2^(emax+1) - ulp, above it).

Readings where the specification leaves a choice open for this path (listed
in the design notes too):
  * a block whose values are all zero gets scale code 0 and element codes 0;
  * inputs are finite fp16, so shared_exp stays inside E8M0's range
    (fp16 magnitudes span 2^-24 .. 65504) and no scale clamping is needed;
  * negative zero is encoded as +0 (sign bit clear) for a zero result.

The product of an MXFP8 row and an MXFP4 column is
  out[m, n] = sum_b X_a[m, b] * X_w[n, b] * sum_{j<32} a[m, 32b+j] * w[n, 32b+j]
formed here in fp64, exact for every size used (each element product needs
at most 4 + 2 significant bits, a block dot at most 17, and the scaled block
terms are summed in fp64).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_EMAX = 8
E4M3_MAX = 448.0
E2M1_EMAX = 2
E2M1_MAX = 6.0


def e4m3_value(code) -> np.ndarray:
    """Value of FP8 E4M3 codes (OCP: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 is subnormal, m * 2^-9; no infinities; S.1111.111 is NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e2m1_value(code) -> np.ndarray:
    """Value of FP4 E2M1 codes (OCP: 1 sign, 2 exponent bits with bias 1, 1 mantissa
    bit; exponent field 0 is subnormal, m * 0.5; no infinities or NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return sign * mag


def _round_minifloat(v: np.ndarray, mant_bits: int, bias: int, max_normal: float, max_code: int) -> np.ndarray:
    """Magnitude code of |v| rounded to a sign-magnitude minifloat with `mant_bits`
    mantissa bits and exponent bias `bias`: nearest, ties to even, clamped to the
    largest normal.  Subnormals (below 2^(1-bias)) have the fixed step 2^(1-bias-mant)."""
    a = np.minimum(np.abs(v.astype(np.float64)), max_normal)
    min_normal_exp = 1 - bias
    step_sub = 2.0 ** (min_normal_exp - mant_bits)
    # subnormal range: integer multiples of step_sub (reaching 2^mant = the smallest normal)
    sub_q = np.rint(a / step_sub)                     # exact scaling by a power of two; rint ties to even
    e = np.frexp(np.where(a > 0, a, 1.0))[1] - 1.0   # floor(log2 a), exactly
    e = np.maximum(e, min_normal_exp)
    frac = a / np.exp2(e) - 1.0                       # in [0, 1) for normal a
    mq = np.rint(frac * (1 << mant_bits))             # ties to even
    carry = mq >= (1 << mant_bits)
    e = np.where(carry, e + 1, e)
    mq = np.where(carry, 0, mq)
    normal_code = ((e + bias).astype(np.int64) << mant_bits) | mq.astype(np.int64)
    code = np.where(a < 2.0 ** min_normal_exp, sub_q.astype(np.int64), normal_code)
    return np.minimum(code, max_code)


def round_e4m3(v) -> np.ndarray:
    """fp8 E4M3 codes of v: nearest, ties to even, saturating at +-448, +0 for zero."""
    v = np.asarray(v, dtype=np.float64)
    mag = _round_minifloat(v, 3, 7, E4M3_MAX, 0x7E)
    return (np.where((v < 0) & (mag != 0), 0x80, 0) | mag).astype(np.uint8)


def round_e2m1(v) -> np.ndarray:
    """fp4 E2M1 codes of v: nearest, ties to even, saturating at +-6, +0 for zero."""
    v = np.asarray(v, dtype=np.float64)
    mag = _round_minifloat(v, 1, 1, E2M1_MAX, 0x7)
    return (np.where((v < 0) & (mag != 0), 0x8, 0) | mag).astype(np.uint8)


def mx_quantize(x16: np.ndarray, elem: str):
    """MX conversion of fp16 rows [R][K] in blocks of 32 along K.

    elem = "e4m3" (MXFP8) or "e2m1" (MXFP4).  Returns (codes uint8 [R][K], one
    element code per byte; scale codes uint8 [R][K/32], X = 2^(code - 127)).
    Parity: pinned by the element tables of the specification, the rounding
    brute force, the shared-exponent rule, exact power-of-two scaling and the
    lossless special case (tests/test_oracle_mx.py).
    """
    x = np.asarray(x16)
    assert x.dtype == np.float16 and x.ndim == 2 and x.shape[1] % BLOCK == 0
    r, k = x.shape
    xb = x.astype(np.float64).reshape(r, k // BLOCK, BLOCK)
    assert np.all(np.isfinite(xb)), "inputs must be finite"
    emax, rnd = (E4M3_EMAX, round_e4m3) if elem == "e4m3" else (E2M1_EMAX, round_e2m1)
    amax = np.max(np.abs(xb), axis=2)
    nz = amax > 0
    # floor(log2(amax)), exactly: frexp gives amax = f * 2^e with f in [0.5, 1)
    shared = np.where(nz, (np.frexp(np.where(nz, amax, 1.0))[1] - 1.0) - emax, -127.0)
    scale_codes = (shared + 127).astype(np.int64)
    assert np.all((scale_codes >= 0) & (scale_codes <= 254))
    scaled = xb / np.exp2(shared)[:, :, None]        # exact: division by a power of two
    codes = rnd(scaled).reshape(r, k)
    return codes, scale_codes.astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scale_codes: np.ndarray, elem: str) -> np.ndarray:
    """Values element * 2^(scale - 127), fp64 [R][K]."""
    val = e4m3_value(codes) if elem == "e4m3" else e2m1_value(codes)
    r, k = codes.shape
    return (val.reshape(r, k // BLOCK, BLOCK) *
            np.exp2(scale_codes.astype(np.float64) - 127.0)[:, :, None]).reshape(r, k)


def mx_linear(x16: np.ndarray, w16: np.ndarray) -> np.ndarray:
    """out [M][N] fp64 = MXFP8(x) . MXFP4(w)^T with per-block scales (see the module doc).

    x16 fp16 [M][K] activations, w16 fp16 [N][K] weights: both are converted
    by mx_quantize, then multiplied by mx_linear_prequantized (one body for
    both entry points).  Parity: pinned by the lossless special case (equals
    np.matmul of the raw inputs) and power-of-two scaling
    (tests/test_oracle_mx.py).
    """
    qa, sa = mx_quantize(x16, "e4m3")
    qw, sw = mx_quantize(w16, "e2m1")
    return mx_linear_prequantized(qa, sa, qw, sw)


def mx_linear_prequantized(qa, sa, qw, sw) -> np.ndarray:
    """The product from codes already converted by mx_quantize: each block term
    is X_a * X_w * (the exact block dot of the element values), summed in fp64.
    mx_linear is this function after the conversions, so its pins cover it."""
    va = e4m3_value(qa).reshape(qa.shape[0], -1, BLOCK)
    vw = e2m1_value(qw).reshape(qw.shape[0], -1, BLOCK)
    dots = np.einsum("mbj,nbj->mnb", va, vw)          # exact block dots (small integers times 2^-k)
    scale = np.exp2(sa.astype(np.float64)[:, None, :] + sw.astype(np.float64)[None, :, :] - 254.0)
    return np.sum(dots * scale, axis=2)


def mx_abs_terms(qa, sa, qw, sw) -> np.ndarray:
    """sum_k |a_k * w_k| of every output (fp64 [M][N]), the magnitude that bounds
    the accumulation error of a reduced-precision dot product."""
    va = np.abs(mx_dequantize(qa, sa, "e4m3"))
    vw = np.abs(mx_dequantize(qw, sw, "e2m1"))
    return va @ vw.T
