"""CPU oracle for decode attention over an fp16 KV cache -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark may import this
module; the GPU library shares no code with it.

The pages' benchmark decodes with an fp16 KV cache at context 640 and keeps
that cache in a GPU-friendly layout (ML Drift explainer on tech.dede.sh,
section "Stage-aware optimization for large language models"; x-techcon
article, section on stage-aware optimisation).  The step between the QKV and
O projections is scaled dot-product attention of the newest token over every
cached position and itself; this oracle is its textbook definition with
grouped query heads (query head h reads KV head h // (Hq / Hkv)):

  K_t = k_past[g, t]  for t < L - 1,   K_{L-1} = fp16(k_new[g])   (V likewise)
  s_t = (q[h] . K_t) / sqrt(D)
  p_t = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
  out[h] = fp16( sum_t p_t V_t )

in fp64 with one final rounding to fp16.  Readings (the pages fix no more
than "fp16 KV cache, context 640"): the query enters in fp32, as the QKV
projection produces it; the new key and value are rounded to fp16 on their way
into the cache and attended in that form; nothing beyond the L positions is
masked.  Layout here is logical ([Hkv][positions][D] for both caches); the
tests map the library's storage order onto it.
"""
from __future__ import annotations

import numpy as np


def _kv(k_new, v_new, k_past, v_past):
    keys = np.concatenate([k_past.astype(np.float64), k_new.astype(np.float16).astype(np.float64)[:, None]], axis=1)
    vals = np.concatenate([v_past.astype(np.float64), v_new.astype(np.float16).astype(np.float64)[:, None]], axis=1)
    return keys, vals   # [Hkv][L][D]


def attention_probs(q: np.ndarray, k_new: np.ndarray, k_past: np.ndarray) -> np.ndarray:
    """Softmax weights p[h][t] (fp64) of every query head over the L = k_past.shape[1] + 1 positions."""
    hq, d = q.shape
    hkv = k_new.shape[0]
    assert hq % hkv == 0 and k_past.shape[0] == hkv and k_past.shape[2] == d
    keys = np.concatenate([k_past.astype(np.float64), k_new.astype(np.float16).astype(np.float64)[:, None]], axis=1)
    group = hq // hkv
    probs = np.empty((hq, keys.shape[1]), np.float64)
    for h in range(hq):
        s = keys[h // group] @ q[h].astype(np.float64) / np.sqrt(d)
        e = np.exp(s - s.max())
        probs[h] = e / e.sum()
    return probs


def decode_attention_exact(q, k_new, v_new, k_past, v_past):
    """(out fp64 [Hq][D] before the final rounding, sum_t p_t |V_t| fp64 [Hq][D])."""
    hq = q.shape[0]
    group = hq // k_new.shape[0]
    _, vals = _kv(k_new, v_new, k_past, v_past)
    p = attention_probs(q, k_new, k_past)
    out = np.stack([p[h] @ vals[h // group] for h in range(hq)])
    mag = np.stack([p[h] @ np.abs(vals[h // group]) for h in range(hq)])
    return out, mag


def decode_attention(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, k_past: np.ndarray,
                     v_past: np.ndarray) -> np.ndarray:
    """q fp32 [Hq][D]; k_new, v_new fp32 [Hkv][D]; k_past, v_past fp16 [Hkv][L-1][D] (L-1 may be 0).
    Returns out fp16 [Hq][D].  Parity: pinned by closed forms (one position, two positions
    through the logistic function, uniform weights giving the mean), invariances (order of
    positions, a common shift of every score), the GQA head mapping and stability at large
    scores (tests/test_oracle_attention.py)."""
    out, _ = decode_attention_exact(q, k_new, v_new, k_past, v_past)
    return out.astype(np.float16)
