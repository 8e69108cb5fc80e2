"""KV-cache size formulas.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存" (m.nxbn.cn),
section on why long context exhausts memory first: KV cache bytes =
2 x layers x kv_heads x head_dim x sequence length x bytes per value.
"""
from __future__ import annotations

from .layout import block_bytes, BLOCK


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, bytes_per_value: float) -> float:
    """The page's formula (no scale or zero-point overhead)."""
    return 2 * layers * kv_heads * head_dim * seq_len * bytes_per_value


def stored_bytes_per_token(fmt: str, head_dim: int = 128) -> float:
    """Bytes one token occupies in this cache's block layout for K and V together,
    including scales / zero points (fp16 residual: 2 bytes per value)."""
    if fmt == "fp16":
        return 2 * head_dim * 2
    return block_bytes(fmt) / BLOCK


def packed_cache_bytes(fmt: str, layers: int, kv_heads: int, seq_len: int, batch: int = 1) -> float:
    """Bytes of a cache of seq_len tokens stored entirely in `fmt` (whole 128-token blocks)."""
    blocks = -(-seq_len // BLOCK)
    return layers * batch * kv_heads * blocks * block_bytes(fmt)
