"""Single-token decode attention over the decoded cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each decode step reads every cached K/V (page "KV Cache量化实战：Model Optimizer为大模型
长上下文省下50%显存" (m.nxbn.cn), section on why long context exhausts memory
first) and the dequantized values take part in attention (page
"NVFP4 KV缓存技术详解" §2.1).  The plainest reading is standard scaled
dot-product attention of one query token:

    s_t = sigma * sum_d q_d * k_hat[t, d]
    p_t = exp(s_t - max s) / sum_t' exp(s_t' - max s)
    out_d = sum_t p_t * v_hat[t, d]

Grouped-query attention: query head h reads kv head h // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, sigma: float) -> np.ndarray:
    """q [G, D] (any float), k_hat/v_hat [T, D] float64 -> out [G, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    s = sigma * (q @ k_hat.T)                       # [G, T]
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v_hat


def decode_layer(layer_cache, q: np.ndarray, sigma: float, b_list=None) -> np.ndarray:
    """Attention for one layer: q fp16 [B, Hq, D] -> float64 [B, Hq, D]
    (only the batch entries in b_list are filled when given; the rest are NaN)."""
    B, Hq, D = q.shape
    H = len(layer_cache.k_hist[0][0])
    G = Hq // H
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if b_list is None else b_list):
        for h in range(H):
            k_hat, v_hat = layer_cache.decoded(b, h)
            out[b, h * G:(h + 1) * G] = attend(q[b, h * G:(h + 1) * G], k_hat, v_hat, sigma)
    return out
