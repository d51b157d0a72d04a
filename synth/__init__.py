"""Seeded synthetic inputs for the W4A8 block-32 linear layer.

This module serves both the CPU oracle and the GPU path, so it holds none of
the method's arithmetic: it draws random numbers, rounds them once to the
storage dtype and returns plain row-major arrays.  No quantisation, packing
or dot product happens here.

Generator: numpy's PCG64, seeded with the pair (config seed, tensor id), so
every tensor of every workload is reproducible on its own.

Workloads (the ML Drift pages' LLM benchmark setup -- prefill 512 tokens,
decode 128, context 640, 4-bit weights in blocks of 32 -- is given on the
tech.dede.sh explainer, section "Stage-aware optimization for large language
models"; the shapes below are a synthetic transformer layer of hidden size
2048 standing in for the trained model, whose weights are not used):

  single   M=1, K=2048, N=2048
  decode   M=1 projections qkv 2048->2560, o 2048->2048,
           gate_up 2048->16384, down 8192->2048
  prefill  the same projections at M=512, activations with outlier channels
  wide     K=4096, N=14336 at M in {1, 4, 8, 16}, outlier channels
  e2e      26 decode layers + a 2048->262144 LM head
"""
from __future__ import annotations

import numpy as np

# Distribution parameters of the synthetic workloads.
W_LO, W_HI = -8, 7              # int4 weight values, uniform, both ends included
SCALE_LO, SCALE_HI = 0.005, 0.02  # fp16 weight scales, uniform
OUTLIER_FRACTION = 0.01         # share of input channels that are outliers
OUTLIER_GAIN = 20.0             # outlier channels are multiplied by this

LAYER_SHAPES = {                # name -> (K, N) of one synthetic decoder layer
    "qkv": (2048, 2560),
    "o": (2048, 2048),
    "gate_up": (2048, 16384),
    "down": (8192, 2048),
}
LM_HEAD_SHAPE = (2048, 262144)
N_LAYERS_E2E = 26
PREFILL_TOKENS = 512
DECODE_TOKENS = 128

WORKLOADS = {
    "single": {"seed": 0, "M": [1], "shapes": {"single": (2048, 2048)}, "outliers": False},
    "decode": {"seed": 1, "M": [1], "shapes": LAYER_SHAPES, "outliers": False},
    "prefill": {"seed": 2, "M": [PREFILL_TOKENS], "shapes": LAYER_SHAPES, "outliers": True},
    "wide": {"seed": 3, "M": [1, 4, 8, 16], "shapes": {"wide": (4096, 14336)}, "outliers": True},
    "e2e": {"seed": 4, "M": [1], "shapes": LAYER_SHAPES, "outliers": True},
}


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    """Independent PCG64 stream for tensor `tensor_id` of workload `seed`."""
    return np.random.Generator(np.random.PCG64([int(seed), int(tensor_id)]))


def int4_values(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 array [n][k] of weight values drawn uniformly from [-8, 7]."""
    return g.integers(W_LO, W_HI + 1, size=(n, k), dtype=np.int8)


def weight_scales(g: np.random.Generator, n: int, k: int, block: int = 32) -> np.ndarray:
    """fp16 array [n][k/block]: fp64 uniform in [0.005, 0.02], one rounding to fp16."""
    return g.uniform(SCALE_LO, SCALE_HI, size=(n, k // block)).astype(np.float16)


def outlier_channels(g: np.random.Generator, k: int) -> np.ndarray:
    """round(1% of k) distinct input channels, sorted (20 at k=2048, 41 at 4096, 82 at 8192)."""
    count = int(round(OUTLIER_FRACTION * k))
    return np.sort(g.choice(k, size=count, replace=False))


def activations(g: np.random.Generator, m: int, k: int, outliers: np.ndarray | None = None) -> np.ndarray:
    """fp16 array [m][k]: fp64 N(0,1), outlier channels times 20 in fp64, one rounding to fp16."""
    x = g.standard_normal(size=(m, k))
    if outliers is not None and len(outliers):
        x[:, outliers] *= OUTLIER_GAIN
    return x.astype(np.float16)


def linear_inputs(seed: int, m: int, k: int, n: int, outliers: bool = False, tensor_base: int = 0):
    """(x fp16 [m][k], qw int8 [n][k], sw fp16 [n][k/32]) for one linear layer.

    Tensor ids: tensor_base+0 weights, +1 scales, +2 activations, +3 outlier channels.
    """
    qw = int4_values(rng(seed, tensor_base + 0), n, k)
    sw = weight_scales(rng(seed, tensor_base + 1), n, k)
    ch = outlier_channels(rng(seed, tensor_base + 3), k) if outliers else None
    x = activations(rng(seed, tensor_base + 2), m, k, ch)
    return x, qw, sw


def workload_inputs(name: str, m: int | None = None):
    """Inputs of every projection of a named workload: {proj: (x, qw, sw)}.

    Projection p (in the order of the workload's shape table) uses tensor ids
    starting at 16*p; the M-sweep of the `wide` workload shares its weights
    and draws activations per M from tensor id 16*p + 4 + M.
    """
    w = WORKLOADS[name]
    mm = w["M"][0] if m is None else m
    out = {}
    for p, (proj, (k, n)) in enumerate(w["shapes"].items()):
        base = 16 * p
        qw = int4_values(rng(w["seed"], base + 0), n, k)
        sw = weight_scales(rng(w["seed"], base + 1), n, k)
        ch = outlier_channels(rng(w["seed"], base + 3), k) if w["outliers"] else None
        x = activations(rng(w["seed"], base + 4 + mm), mm, k, ch)
        out[proj] = (x, qw, sw)
    return out


def e2e_layer_weights(layer: int) -> dict:
    """int4 weights and fp16 scales of decoder layer `layer` of the end-to-end workload:
    {proj: (qw int8 [N][K], sw fp16 [N][K/32])}; tensor ids 64*layer + 2p (+1 for scales)."""
    seed = WORKLOADS["e2e"]["seed"]
    out = {}
    for p, (proj, (k, n)) in enumerate(LAYER_SHAPES.items()):
        base = 64 * layer + 2 * p
        out[proj] = (int4_values(rng(seed, base), n, k), weight_scales(rng(seed, base + 1), n, k))
    return out


def e2e_head_weights():
    """The 2048 -> 262144 LM head of the end-to-end workload (tensor ids 1_000_000, +1)."""
    seed = WORKLOADS["e2e"]["seed"]
    k, n = LM_HEAD_SHAPE
    return int4_values(rng(seed, 1_000_000), n, k), weight_scales(rng(seed, 1_000_001), n, k)


def e2e_prompt() -> np.ndarray:
    """The 512 prefill rows of the end-to-end workload: fp16 N(0,1) with outlier channels
    (tensor ids 2_000_000 for the activations, 2_000_001 for the channels)."""
    seed = WORKLOADS["e2e"]["seed"]
    k = LM_HEAD_SHAPE[0]
    ch = outlier_channels(rng(seed, 2_000_001), k)
    return activations(rng(seed, 2_000_000), PREFILL_TOKENS, k, ch)


# Decode attention of the synthetic layer: the QKV projection's 2560 outputs read as
# 8 query heads of 256, one key head and one value head (2048 + 256 + 256), over an
# fp16 KV cache of the pages' context of 640 positions (512 prefill + 128 decode).
ATTN_HEADS = 8
ATTN_KV_HEADS = 1
ATTN_HEAD_DIM = 256
CONTEXT = PREFILL_TOKENS + DECODE_TOKENS
ATTN_Q_GAIN = 2.0   # query scale: scores about N(0, 4), so weight spreads over tens of positions
WORKLOADS["attention"] = {"seed": 5, "M": [1], "shapes": {}, "outliers": False}


def attention_inputs(seed: int, hq: int, hkv: int, d: int, length: int, q_gain: float = ATTN_Q_GAIN):
    """Inputs of one decode-attention step over `length` positions (the newest included):
    q fp32 [hq][d] = q_gain * N(0,1); k_new, v_new fp32 [hkv][d] = N(0,1);
    k_past, v_past fp16 [hkv][length-1][d] = N(0,1) rounded once.  Tensor ids 0 .. 4."""
    q = (rng(seed, 0).standard_normal((hq, d)) * q_gain).astype(np.float32)
    k_new = rng(seed, 1).standard_normal((hkv, d)).astype(np.float32)
    v_new = rng(seed, 2).standard_normal((hkv, d)).astype(np.float32)
    k_past = rng(seed, 3).standard_normal((hkv, length - 1, d)).astype(np.float16)
    v_past = rng(seed, 4).standard_normal((hkv, length - 1, d)).astype(np.float16)
    return q, k_new, v_new, k_past, v_past
