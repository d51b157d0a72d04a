"""CPU oracle for the W4A8 block-32 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The GPU library never calls it and shares no code
with it; the two meet only on the seeded inputs of `synth`.

What the pages fix (ML Drift explainer on tech.dede.sh, section "Stage-aware
optimization for large language models"; x-techcon article, section on moving
less data for large models): weights are 4-bit in blocks of 32, and in the
decode stage the kernel quantises activations itself.  Everything else is
this implementation's pinned reading of those two statements:

  * weights: symmetric int4 qw in [-8, 7], one fp16 scale sw per output
    column per 32 consecutive input elements, dequantised value qw * sw;
  * activations: per token row, per 32 consecutive input elements,
    sx = fp32(max|x| / 127), qx = clamp(round_half_even(fp32(x / sx)), -127, 127),
    and an all-zero block gives sx = 0, qx = 0;
  * output: out[m, n] = sum_b sx[m, b] * sw[n, b] * I[m, n, b] with the exact
    integer block dot I[m, n, b] = sum_{j<32} qx[m, 32b+j] * qw[n, 32b+j].

The quantisation decisions (a division, then a rounding to an integer) are
taken in fp32, the GPU kernel's precision, because the pages fix none; the
scaled sum is formed in fp64 and is exact up to the final rounding for every
size used here (I*sw needs 26 bits, times sx 50 bits, both below 53).

Every function here is plain numpy, without blocking or reordering beyond the
definition above.  oracle/w4a8_ref.c (bound by oracle/cref.py) computes the
same linear in plain C for timing on the host cores; the tests hold it to this
module bit for bit.  Parity status of each function is stated in its docstring;
the pins live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32          # input elements per quantisation block (weights and activations)
QMAX_ACT = 127      # symmetric int8 range used for activations


def quantize_activations(x16: np.ndarray):
    """Per-(row, block) int8 quantisation of fp16 activations.

    Returns (qx int8 [M][K], sx float32 [M][K/32]).  Steps, per row m and
    block b of 32 consecutive elements:
      amax = max_j |x|              (exact; fp16 -> fp32 widening is exact)
      sx   = fp32(amax / 127)       (IEEE round-to-nearest division)
      qx_j = clamp(rint(fp32(x_j / sx)), -127, 127), rint rounding half to even
      amax == 0  ->  sx = 0, qx = 0
    Inputs must be finite.  Pinned by: hand-derived blocks in
    tests/golden/quant_blocks.json, the rounding-error bound, the amax element
    reaching +-127, exact power-of-two scaling invariance.
    """
    x = np.asarray(x16)
    assert x.dtype == np.float16 and x.ndim == 2 and x.shape[1] % BLOCK == 0
    m, k = x.shape
    xb = x.astype(np.float32).reshape(m, k // BLOCK, BLOCK)
    assert np.all(np.isfinite(xb)), "activations must be finite"
    amax = np.max(np.abs(xb), axis=2)                       # float32 [M][B]
    sx = (amax / np.float32(QMAX_ACT)).astype(np.float32)   # fp32 division
    nonzero = sx > 0
    divisor = np.where(nonzero, sx, np.float32(1.0)).astype(np.float32)
    ratio = (xb / divisor[:, :, None]).astype(np.float32)   # fp32 division
    q = np.clip(np.rint(ratio), -QMAX_ACT, QMAX_ACT)        # half to even
    q = np.where(nonzero[:, :, None], q, 0.0)
    return q.astype(np.int8).reshape(m, k), sx


def pack_weights(qw: np.ndarray, sw16: np.ndarray):
    """Pack int4 weights into the K-block-major layout used by the library.

    qw int8 [N][K] in [-8, 7], sw16 fp16 [N][K/32]  ->
      packed   uint8 [K/32][N][16]: byte j of (block b, column n) holds
               element 32b+j in its low nibble and element 32b+16+j in its
               high nibble, both as 4-bit two's complement;
      w_scales fp16  [K/32][N]:     w_scales[b, n] = sw16[n, b].
    Pinned by the hand-derived bytes in tests/golden/pack_layout.json and a
    round trip through `unpack_weights` over every nibble value and position.
    """
    q = np.asarray(qw)
    assert q.dtype == np.int8 and q.ndim == 2 and q.shape[1] % BLOCK == 0
    assert q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    n, k = q.shape
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8).reshape(n, k // BLOCK, BLOCK)
    lo = nib[:, :, :16]
    hi = nib[:, :, 16:]
    packed = (lo | (hi << 4)).astype(np.uint8)               # [N][B][16]
    packed = np.ascontiguousarray(packed.transpose(1, 0, 2))  # [B][N][16]
    w_scales = np.ascontiguousarray(np.asarray(sw16, dtype=np.float16).T)
    return packed, w_scales


def unpack_weights(packed: np.ndarray, w_scales: np.ndarray):
    """Inverse of `pack_weights`: returns (qw int8 [N][K], sw16 fp16 [N][K/32])."""
    p = np.asarray(packed, dtype=np.uint8)
    nb, n, width = p.shape
    assert width == 16
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    blocks = np.concatenate([lo, hi], axis=2)                 # [B][N][32]
    qw = blocks.transpose(1, 0, 2).reshape(n, nb * BLOCK).astype(np.int8)
    return qw, np.ascontiguousarray(np.asarray(w_scales, dtype=np.float16).T)


def block_sums(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """Exact integer block dot products, int64 [M][N][K/32].

    I[m, n, b] = sum_{j<32} qx[m, 32b+j] * qw[n, 32b+j].  Each block is one
    fp64 matrix product of integer-valued operands: every product and
    partial sum is an integer of magnitude <= 32*127*8 < 2**53, so the fp64
    product is exact and converts back to int64 without loss.  Pinned by
    brute-force integer loops on tiny shapes and by the integer-GEMM special
    case (K = 32, unit scales).
    """
    a = np.asarray(qx)
    w = np.asarray(qw)
    m, k = a.shape
    n = w.shape[0]
    nb = k // BLOCK
    out = np.empty((m, n, nb), dtype=np.int64)
    af = a.astype(np.float64).reshape(m, nb, BLOCK)
    wf = w.astype(np.float64).reshape(n, nb, BLOCK)
    for b in range(nb):
        out[:, :, b] = (af[:, b, :] @ wf[:, b, :].T).astype(np.int64)
    return out


def scale_block_sums(sums: np.ndarray, sx: np.ndarray, sw16: np.ndarray) -> np.ndarray:
    """out[m, n] = sum_b sums[m, n, b] * sw[n, b] * sx[m, b], in fp64 [M][N].

    Blocks are summed in ascending order.  Pinned against a dequantise-then-
    fp64-matmul brute force on tiny shapes and hand-derived examples in
    tests/golden/linear_examples.json.
    """
    s = np.asarray(sums, dtype=np.float64)
    swd = np.asarray(sw16, dtype=np.float16).astype(np.float64)   # [N][B]
    sxd = np.asarray(sx, dtype=np.float32).astype(np.float64)     # [M][B]
    out = np.zeros(s.shape[:2], dtype=np.float64)
    for b in range(s.shape[2]):
        out += s[:, :, b] * swd[None, :, b] * sxd[:, b, None]
    return out


def linear(x16: np.ndarray, qw: np.ndarray, sw16: np.ndarray) -> np.ndarray:
    """W4A8 block-32 linear: quantise x, integer block dots, fp64 scaled sum.

    x16 fp16 [M][K], qw int8 [N][K], sw16 fp16 [N][K/32] -> fp64 [M][N].
    """
    qx, sx = quantize_activations(x16)
    return scale_block_sums(block_sums(qx, qw), sx, sw16)


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest value per row, lowest index on ties; -0.0 == +0.0.

    The pages' benchmark samples with argmax (ML Drift explainer, section
    "Stage-aware optimization for large language models"); the tie rule is
    this implementation's choice.  Inputs must be finite.  Pinned against a
    brute-force scan with constructed ties and signed zeros.
    """
    v = np.asarray(logits)
    assert np.all(np.isfinite(v))
    return np.argmax(v, axis=-1)


# ---------------------------------------------------------------------------
# Synthetic decoder layer around the linear, for the end-to-end workload (the
# pages' benchmark: prefill 512 / decode 128, argmax sampling, sync every
# token -- ML Drift explainer on tech.dede.sh, section "Stage-aware
# optimization for large language models").  The wiring is this
# implementation's stand-in for a transformer layer without attention; x is an
# fp32 residual stream, every linear output is an fp32 tensor:
#   n1 = fp16(x / rms(x)); q = L(n1; qkv); a = fp16(q[:, :H]); o = L(a; o)
#   x = x + s*o; n2 = fp16(x / rms(x)); g = L(n2; gate_up)
#   u = fp16(g[:, :F] * g[:, F:]); d = L(u; down); x = x + s*d
# ---------------------------------------------------------------------------

def rms_norm_fp16(x32: np.ndarray, eps: float) -> np.ndarray:
    """fp16(x / sqrt(mean(x^2) + eps)) per row, in fp64 before the one rounding to fp16.

    Pinned by constant rows (closed form), exact power-of-two invariance with
    eps = 0, and the unit mean square of the result.
    """
    xd = np.asarray(x32, dtype=np.float32).astype(np.float64)
    ms = np.mean(xd * xd, axis=1, keepdims=True)
    return (xd / np.sqrt(ms + eps)).astype(np.float16)


def residual_add(x32: np.ndarray, d32: np.ndarray, alpha: float) -> np.ndarray:
    """fp32(x + alpha * d) with alpha taken as fp32 and one rounding (an fma).

    Exact in fp64 before the rounding (fp32 x fp32 products and their sums with
    fp32 values fit in 53 bits here).  Pinned against exact rational arithmetic.
    """
    a = np.float64(np.float32(alpha))
    return (np.asarray(x32, np.float32).astype(np.float64) +
            a * np.asarray(d32, np.float32).astype(np.float64)).astype(np.float32)


def gated_fp16(g32: np.ndarray) -> np.ndarray:
    """fp16(fp32(g[:, :F] * g[:, F:])) with F = half the row; pinned by a hand example."""
    g = np.asarray(g32, dtype=np.float32)
    f = g.shape[1] // 2
    return (g[:, :f] * g[:, f:]).astype(np.float32).astype(np.float16)


def linear_fp32(x16, qw, sw16) -> np.ndarray:
    """The linear's output as the fp32 tensor it is stored in."""
    return linear(x16, qw, sw16).astype(np.float32)


def decoder_layer(x32: np.ndarray, w: dict, residual_scale: float, eps: float) -> np.ndarray:
    """One layer of the wiring above; w maps qkv/o/gate_up/down to (qw int8 [N][K], sw fp16)."""
    x = np.asarray(x32, dtype=np.float32).copy()
    h = x.shape[1]
    n1 = rms_norm_fp16(x, eps)
    q = linear_fp32(n1, *w["qkv"])
    a = q[:, :h].astype(np.float16)
    o = linear_fp32(a, *w["o"])
    x = residual_add(x, o, residual_scale)
    n2 = rms_norm_fp16(x, eps)
    g = linear_fp32(n2, *w["gate_up"])
    u = gated_fp16(g)
    d = linear_fp32(u, *w["down"])
    return residual_add(x, d, residual_scale)
