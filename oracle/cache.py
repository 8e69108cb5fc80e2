"""Residual + tier schedule of one layer's cache, and the stored bytes it produces.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Residual cache -- page "KV缓存量化技术：提升大模型长文本生成效率" (rkmt.cn) §2.2: two
buffers, a quantized main cache and an FP16 residual holding the most recent
R = 128 tokens; when the residual is full its contents are quantized, merged
into the main cache and the residual is cleared.  The configuration names
(nbits, group_size, residual_length) follow the same page §3.2.

Readings (listed in the design notes):
  * the flush is lazy: tokens arrive one at a time, in order; a token arriving
    while the residual already holds R tokens first flushes those R tokens;
  * R = 0 quantizes every token as it arrives (the NVFP4 update step of page
    "NVFP4 KV缓存技术详解" §2.1: quantize the new token and append it);
  * an explicit flush quantizes the r (1..R) tokens currently held;
  * memory compression by age (rkmt.cn §4.2: stronger quantization such as INT2
    for early blocks): every group of tokens quantized together (a "chunk":
    a flushed residual, or a single token when R = 0) is stored in the old-tier
    format when old_after > 0 and all of its tokens are at least old_after
    positions behind the length the cache reaches at the end of the append
    call that quantizes it (chunk end <= L1 - old_after); otherwise in the
    young-tier format.  A stored token is never re-quantized.
  * each tier is an append-only sequence of 128-slot blocks, filled in the
    order chunks are quantized.
  * age-based demotion (optional; the same §4.2 passage read as tokens growing
    old while decoding): at the end of every append or flush, while the first
    live young block is full and its last token is at least old_after
    positions behind the length, the block moves to the old tier: its 128
    tokens are appended to the old tier in slot order, quantized in the old
    format from the fp16 rounding (to nearest even, saturating at +-65504) of
    their young decoded values, since the fp16 inputs are no longer kept.  The young tier then
    starts one block later.
"""
from __future__ import annotations

import numpy as np

from .quant import quantize_tokens, dequantize_tokens
from .numerics import f16_saturate
from .layout import pack_arena, pack_residual, BLOCK


class Schedule:
    """Token bookkeeping for one layer (the same for every batch entry and kv head)."""

    def __init__(self, residual_len: int, old_after: int = 0, demote: bool = False):
        self.R = residual_len
        self.old_after = old_after
        self.demote = demote
        self.length = 0
        self.residual: list[int] = []     # stream positions, oldest first
        self.young: list[int] = []        # every token ever quantized young, in slot order
        self.young_head = 0               # young slots before this one were demoted
        self.old: list[int] = []
        self.old_demoted: list[bool] = [] # per old slot: came from the young tier
        self.flushes = 0

    def _old_extend(self, chunk: list[int], demoted: bool):
        self.old.extend(chunk)
        self.old_demoted.extend([demoted] * len(chunk))

    def _demote(self):
        while (self.demote and self.old_after > 0 and self.young_head + BLOCK <= len(self.young)
               and self.young[self.young_head + BLOCK - 1] + 1 <= self.length - self.old_after):
            self._old_extend(self.young[self.young_head:self.young_head + BLOCK], True)
            self.young_head += BLOCK

    def live_young(self) -> list[int]:
        return self.young[self.young_head:]

    def _quantize_chunk(self, chunk: list[int], L1: int):
        if self.old_after > 0 and chunk[-1] + 1 <= L1 - self.old_after:
            self._old_extend(chunk, False)
        else:
            self.young.extend(chunk)

    def append(self, n: int):
        L1 = self.length + n
        for p in range(self.length, L1):
            if self.R > 0:
                if len(self.residual) == self.R:
                    self._quantize_chunk(self.residual, L1)
                    self.residual = []
                    self.flushes += 1
                self.residual.append(p)
            else:
                self._quantize_chunk([p], L1)
        self.length = L1
        self._demote()

    def flush(self):
        if self.residual:
            self._quantize_chunk(self.residual, self.length)
            self.residual = []
            self.flushes += 1
        self._demote()


class LayerCache:
    """One layer's cache for all (batch, kv_head): the schedule plus the fp16 history."""

    def __init__(self, fmt: str, residual_len: int, old_fmt: str | None = None, old_after: int = 0,
                 demote: bool = False):
        self.fmt = fmt
        self.old_fmt = old_fmt if old_fmt is not None else fmt
        self.sched = Schedule(residual_len, old_after, demote)
        self.k_hist: list[np.ndarray] = []   # fp16 [B, H, n, 128] chunks in stream order
        self.v_hist: list[np.ndarray] = []

    def append(self, k16: np.ndarray, v16: np.ndarray):
        assert k16.shape == v16.shape and k16.dtype == np.float16
        self.k_hist.append(k16)
        self.v_hist.append(v16)
        self.sched.append(k16.shape[2])

    def flush(self):
        self.sched.flush()

    def history(self, b: int, h: int):
        K = np.concatenate([c[b, h] for c in self.k_hist], axis=0)
        V = np.concatenate([c[b, h] for c in self.v_hist], axis=0)
        return K, V

    def tier_tokens(self, tier: str) -> list[int]:
        return {"young": self.sched.live_young(), "old": self.sched.old}[tier]

    def tier_format(self, tier: str) -> str:
        return self.fmt if tier == "young" else self.old_fmt

    def tier_inputs(self, b: int, h: int, tier: str) -> tuple[np.ndarray, np.ndarray]:
        """fp16 [N, 128] K and V that a tier's slots were quantized from: the tokens themselves,
        or for demoted old slots the fp16 rounding of their young decoded values."""
        K, V = self.history(b, h)
        pos = np.asarray(self.tier_tokens(tier), dtype=np.int64)
        k, v = K[pos].copy(), V[pos].copy()
        if tier == "old" and any(self.sched.old_demoted):
            dem = np.asarray(self.sched.old_demoted)
            y = self.fmt
            k[dem] = f16_saturate(dequantize_tokens(quantize_tokens(k[dem], y, "k"), y, "k"))
            v[dem] = f16_saturate(dequantize_tokens(quantize_tokens(v[dem], y, "v"), y, "v"))
        return k, v

    def arena(self, b: int, h: int, tier: str) -> np.ndarray:
        """Packed bytes of one tier for (b, h): uint8 [ceil(N/128), block_bytes]."""
        k, v = self.tier_inputs(b, h, tier)
        fmt = self.tier_format(tier)
        return pack_arena(fmt, quantize_tokens(k, fmt, "k"), quantize_tokens(v, fmt, "v"))

    def residual(self, b: int, h: int) -> tuple[np.ndarray, np.ndarray]:
        K, V = self.history(b, h)
        pos = np.asarray(self.sched.residual, dtype=np.int64)
        return pack_residual(K[pos], V[pos], self.sched.R)

    def decoded(self, b: int, h: int) -> tuple[np.ndarray, np.ndarray]:
        """float64 [L, 128] K_hat, V_hat over every cached token (tiers decoded, residual as fp16)."""
        K, V = self.history(b, h)
        ks, vs = [], []
        for tier in ("old", "young"):
            if len(self.tier_tokens(tier)):
                fmt = self.tier_format(tier)
                k, v = self.tier_inputs(b, h, tier)
                ks.append(dequantize_tokens(quantize_tokens(k, fmt, "k"), fmt, "k"))
                vs.append(dequantize_tokens(quantize_tokens(v, fmt, "v"), fmt, "v"))
        pos = np.asarray(self.sched.residual, dtype=np.int64)
        if pos.size:
            ks.append(K[pos].astype(np.float64))
            vs.append(V[pos].astype(np.float64))
        return np.concatenate(ks), np.concatenate(vs)


def blocks_for(n_tokens: int) -> int:
    return (n_tokens + BLOCK - 1) // BLOCK
