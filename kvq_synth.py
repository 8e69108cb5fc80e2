"""Seeded synthetic inputs (K, V, Q) shared by the tests, the bench and the smoke run.

This module only draws random numbers and casts them to fp16; it holds none of
the quantization or attention arithmetic.  Both the CPU oracle and the GPU path
receive the arrays it returns.

Recipe (one stream per purpose so that layers and steps are independent):
  Generator(PCG64(SeedSequence([1000 + config_id, layer, stream, step])))
  stream 0 = K prefill, 1 = V prefill, 2 = Q, 3 = K append, 4 = V append,
  5 = choice of outlier channels (fixed per (layer, kv_head) for all tokens).
Values are drawn in float64 and cast to fp16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import numpy as np

HEAD_DIM = 128

STREAM_K, STREAM_V, STREAM_Q, STREAM_K_APPEND, STREAM_V_APPEND, STREAM_OUTLIER = range(6)


@dataclasses.dataclass(frozen=True)
class KDist:
    """How K is drawn: 'normal' or 'student_t', with outlier channels scaled by `scale`."""
    kind: str = "normal"
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    nu: float = 4.0


def rng(config_id: int, layer: int, stream: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + config_id, layer, stream, step])))


def outlier_channels(config_id: int, layer: int, num_kv_heads: int, k: int) -> np.ndarray:
    """[num_kv_heads, k] channel indices, drawn without replacement per kv head."""
    g = rng(config_id, layer, STREAM_OUTLIER)
    if k == 0:
        return np.zeros((num_kv_heads, 0), dtype=np.int64)
    return np.stack([g.choice(HEAD_DIM, k, replace=False) for _ in range(num_kv_heads)])


def draw_k(config_id: int, layer: int, batch: int, num_kv_heads: int, n: int, dist: KDist,
           stream: int = STREAM_K, step: int = 0) -> np.ndarray:
    """fp16 [batch, num_kv_heads, n, HEAD_DIM]."""
    g = rng(config_id, layer, stream, step)
    shape = (batch, num_kv_heads, n, HEAD_DIM)
    if dist.kind == "normal":
        x = g.standard_normal(shape, dtype=np.float64)
    elif dist.kind == "student_t":
        x = g.standard_t(dist.nu, size=shape)
    else:
        raise ValueError(dist.kind)
    if dist.outlier_channels:
        ch = outlier_channels(config_id, layer, num_kv_heads, dist.outlier_channels)
        for h in range(num_kv_heads):
            x[:, h, :, ch[h]] *= dist.outlier_scale
    return x.astype(np.float16)


def draw_v(config_id: int, layer: int, batch: int, num_kv_heads: int, n: int,
           stream: int = STREAM_V, step: int = 0) -> np.ndarray:
    g = rng(config_id, layer, stream, step)
    return g.standard_normal((batch, num_kv_heads, n, HEAD_DIM), dtype=np.float64).astype(np.float16)


def draw_q(config_id: int, layer: int, batch: int, num_q_heads: int, step: int = 0) -> np.ndarray:
    """fp16 [batch, num_q_heads, HEAD_DIM], N(0,1)/sqrt(128)."""
    g = rng(config_id, layer, STREAM_Q, step)
    x = g.standard_normal((batch, num_q_heads, HEAD_DIM), dtype=np.float64) / np.sqrt(HEAD_DIM)
    return x.astype(np.float16)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the five workloads: shapes, formats and distributions."""
    config_id: int
    name: str
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    prefill: int
    fmt: str             # young tier: 'int2' | 'int4' | 'int8' | 'nvfp4'
    residual_len: int
    kdist: KDist
    old_fmt: str | None = None
    old_after: int = 0
    decode_steps: int = 1
    append_per_step: int = 0


WORKLOADS = {
    1: Workload(1, "single-layer GQA4 1K int4", 1, 1, 32, 8, 1152, "int4", 128,
                KDist("normal", 4, 15.0)),
    2: Workload(2, "llama2-7b-shaped MHA 1K int4", 32, 4, 32, 32, 1024, "int4", 128,
                KDist("normal", 4, 15.0), append_per_step=128),
    3: Workload(3, "llama3-70b-shaped GQA8 32K nvfp4", 80, 8, 64, 8, 32768, "nvfp4", 0,
                KDist("normal", 3, 20.0)),
    4: Workload(4, "long-context GQA4 128K int4", 32, 8, 32, 8, 131072, "int4", 128,
                KDist("student_t"), decode_steps=64, append_per_step=1),
    5: Workload(5, "256K prefill int2/int4 tiers", 32, 1, 32, 8, 262144, "int4", 128,
                KDist("normal", 4, 10.0), old_fmt="int2", old_after=65536,
                decode_steps=16, append_per_step=1),
}
