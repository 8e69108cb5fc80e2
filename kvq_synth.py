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


# ----------------------------------------------------------------------------- device-side draws
# The full-size workloads hold up to 4.3 GB of fp16 K/V per layer; drawing them on the host
# would take minutes, so the bench and the full-size tests draw them on the GPU with torch's
# seeded generator.  Same recipe (one seed per (config, layer, stream, step), outlier channels
# from the host generator above), a different random stream: these arrays are not equal to
# the host draws, and a test that checks them copies the slices it needs to the host.

DEV_CHUNK_TOKENS = 8192


def torch_seed(config_id: int, layer: int, stream: int, step: int = 0) -> int:
    s = np.random.SeedSequence([1000 + config_id, layer, stream, step]).generate_state(1, dtype=np.uint64)[0]
    return int(s) & ((1 << 63) - 1)


def _dev_gen(config_id, layer, stream, step, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(config_id, layer, stream, step))
    return g


def _dev_fill(out, g, dist: "KDist | None", mult=None):
    """Fill fp16 out [B, H, n, 128] chunk by chunk along tokens from generator g; `mult`
    ([1, H, 1, 128] fp32, outlier channel factors) is applied before the single fp16 rounding."""
    import torch
    B, H, n, D = out.shape
    for t0 in range(0, n, DEV_CHUNK_TOKENS):
        t1 = min(n, t0 + DEV_CHUNK_TOKENS)
        shape = (B, H, t1 - t0, D)
        x = torch.randn(shape, generator=g, device=out.device, dtype=torch.float32)
        if dist is not None and dist.kind == "student_t":
            # Student-t with integer nu: N(0,1) / sqrt(chi2_nu / nu), chi2_nu a sum of nu squared normals
            nu = int(dist.nu)
            assert nu == dist.nu and nu >= 1
            chi = torch.zeros(shape, device=out.device, dtype=torch.float32)
            for _ in range(nu):
                chi.addcmul_(y := torch.randn(shape, generator=g, device=out.device, dtype=torch.float32), y)
            x.div_(torch.sqrt(chi.div_(nu)))
        if mult is not None:
            x.mul_(mult)
        out[:, :, t0:t1] = x.to(torch.float16)


def draw_k_dev(config_id: int, layer: int, batch: int, num_kv_heads: int, n: int, dist: KDist,
               stream: int = STREAM_K, step: int = 0, device="cuda"):
    """fp16 device tensor [batch, num_kv_heads, n, HEAD_DIM] (K, outlier channels scaled)."""
    import torch
    out = torch.empty((batch, num_kv_heads, n, HEAD_DIM), dtype=torch.float16, device=device)
    m = None
    if dist.outlier_channels:
        ch = outlier_channels(config_id, layer, num_kv_heads, dist.outlier_channels)
        mult = np.ones((num_kv_heads, HEAD_DIM), np.float32)
        for h in range(num_kv_heads):
            mult[h, ch[h]] = dist.outlier_scale
        m = torch.from_numpy(mult).to(device)[None, :, None, :]
    _dev_fill(out, _dev_gen(config_id, layer, stream, step, device), dist, m)
    return out


def draw_v_dev(config_id: int, layer: int, batch: int, num_kv_heads: int, n: int,
               stream: int = STREAM_V, step: int = 0, device="cuda"):
    import torch
    out = torch.empty((batch, num_kv_heads, n, HEAD_DIM), dtype=torch.float16, device=device)
    _dev_fill(out, _dev_gen(config_id, layer, stream, step, device), None)
    return out


def draw_q_dev(config_id: int, layer: int, batch: int, num_q_heads: int, step: int = 0, device="cuda"):
    import torch
    g = _dev_gen(config_id, layer, STREAM_Q, step, device)
    x = torch.randn((batch, num_q_heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return (x / np.sqrt(HEAD_DIM)).to(torch.float16)
