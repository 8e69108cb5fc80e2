"""Group quantizers, written from the pages' definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Affine (asymmetric) quantization -- page "KV缓存量化技术：提升大模型长文本生成效率"
(rkmt.cn/news/1711363) §2.1: S = (max - min) / (2^n - 1), Z = round(-min / S),
one (S, Z) per group of 64 elements, codes stored as n-bit integers.  The same page's §4.3
debugging configuration uses groups of 32 (and a 256-token residual); groups of 32, 64 and 128
contiguous head_dim values are supported, named "int4g32", "int4" (64) and "int4g128".  The
same §2.1 lists per-channel quantization among the scheme's options: "int4kc" quantizes K per
channel -- each dim's values over a window of 128 consecutive tokens form one group (the
residual fills and flushes in whole windows) -- and V per token in groups of 64.  The page
prints the code as round(X/S) - Z; with Z = round(-min/S) that sends min to
about -2Z, outside [0, 2^n - 1].  The reading adopted here is the one under which
codes land in [0, 2^n - 1]:

    q = clamp(round(x / S) + Z, 0, 2^n - 1),      x_hat = S * (q - Z)

Readings of what the page leaves open (each listed in the design notes):
  * "round" is round-half-to-even, applied to the exact quotient;
  * S is rounded once from the exact (max - min) / (2^n - 1) to fp16;
  * Z is the exact round(-min / S) using the stored fp16 S, stored as fp16
    (exact for |Z| <= 2048, saturated to +-65504, zero stored as +0);
  * codes use the stored S and stored Z;
  * a group with max == min, or whose S rounds to 0, uses S = |min| (1 when
    min is 0), which makes a constant group decode exactly.

Float64 evaluation decides every rounding exactly here: mx - mn of two fp16
values is exact in float64, and the float64 quotients x/S, -mn/S and
(mx-mn)/(2^n-1) lie further from any rounding boundary of the target (an
integer-plus-half, or an fp16 midpoint) than float64's relative error 2^-53;
the tests pin this against exact rational arithmetic.

FP8 -- page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存", section on the KV
cache formats (an FP8 cast with a fixed scale is the default format): every value is
cast to E4M3 with scale 1, round to nearest even, saturating at 448, sign kept;
decode x_hat = e4m3(code).

FP16 -- the unquantized reference: the pages' comparisons take the fp16 cache as the baseline
(page "KV缓存量化技术：提升大模型长文本生成效率" §3.1, first row of the quality/memory table;
page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存", formats section, keeping
the 16-bit cache).  The stored fields are the fp16 bit patterns themselves; x_hat = x.

MXFP4 -- page "NVFP4 KV缓存技术详解" §3.2 compares NVFP4 with MXFP4 without defining it; the
definition taken is the open microscaling (MX) format's: 32 contiguous head_dim values share a
power-of-two scale X = 2^(floor(log2 amax) - 2) stored as an E8M0 byte (2 is the exponent of
E2M1's largest magnitude, 6 = 1.5 * 2^2), code = sign bit * 8 + E2M1_RNE(min(|x| / X, 6))
(amax / X lies in [4, 8), so values above 6X saturate), decode x_hat = e2m1(code) * X.  A block
of zeros stores byte 0 (the smallest scale) and signed-zero codes.

NVFP4 -- page "NVFP4 KV缓存技术详解" (glsqs.com/news/814573) §2.1 (16 values share
one FP8 scale) and §4.2 (clip range up to 6.0): per 16 contiguous head_dim
values, s = E4M3_RNE(amax / 6) saturating at 448, code = sign bit * 8 +
E2M1_RNE(min(|x| / s, 6)); decode x_hat = e2m1(code) * s.
"""
from __future__ import annotations

import re

import numpy as np

from .numerics import (f16, f16_saturate, e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode, e4m3_cast,
                       e8m0_decode, floor_log2)

GROUP = 64
NV_BLOCK = 16
MX_BLOCK = 32
E2M1_EMAX = 2            # exponent of E2M1's largest magnitude, 6 = 1.5 * 2^2


KC_WINDOW = 128         # tokens per per-channel K group


def affine_params(fmt: str):
    """(code bits, group size along head_dim) of an affine format name ("int4", "int2g32",
    "int8g128", "int4kc": V in groups of 64), else None."""
    m = re.fullmatch(r"int([248])(?:g(32|64|128)|kc)?", fmt)
    if not m:
        return None
    return int(m.group(1)), int(m.group(2) or GROUP)


def k_per_channel(fmt: str) -> bool:
    return fmt.endswith("kc") and affine_params(fmt) is not None


def affine_quantize(x16: np.ndarray, nbits: int):
    """Quantize groups along the last axis (one group per row of the last axis).

    x16: fp16 [..., g].  Returns (codes uint8 [..., g], S fp16 [...], Z fp16 [...]).
    """
    if nbits not in (2, 4, 8):
        raise ValueError(nbits)
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    assert x.shape[-1] in (32, 64, 128)
    qmax = (1 << nbits) - 1
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    S = f16((mx - mn) / qmax)
    degenerate = (mx == mn) | (S == 0)
    S_deg = np.where(mn != 0, f16(np.abs(mn)), np.float16(1.0))
    S = np.where(degenerate, S_deg, S).astype(np.float16)
    S64 = S.astype(np.float64)
    Z = np.rint(-mn / S64)
    Zs = f16_saturate(Z)
    q = np.rint(x / S64[..., None]) + Zs.astype(np.float64)[..., None]
    q = np.clip(q, 0, qmax).astype(np.uint8)
    return q, S, Zs


def affine_dequantize(q: np.ndarray, S: np.ndarray, Z: np.ndarray) -> np.ndarray:
    """x_hat = S * (q - Z) in float64 (exact: S and Z are fp16, q a small integer)."""
    return S.astype(np.float64)[..., None] * (q.astype(np.float64) - Z.astype(np.float64)[..., None])


def nvfp4_quantize(x16: np.ndarray):
    """Quantize blocks of 16 along the last axis.

    x16: fp16 [..., 16].  Returns (codes uint8 [..., 16] in 0..15, scale byte uint8 [...]).
    """
    x = np.asarray(x16, dtype=np.float16)
    assert x.shape[-1] == NV_BLOCK
    amax = np.abs(x.astype(np.float64)).max(axis=-1)
    sbyte = e4m3_encode(amax / 6.0)
    s = e4m3_decode(sbyte)
    codes = e2m1_encode(x, s[..., None])
    return codes, sbyte


def nvfp4_dequantize(codes: np.ndarray, sbyte: np.ndarray) -> np.ndarray:
    return e2m1_decode(codes) * e4m3_decode(sbyte)[..., None]


def mxfp4_quantize(x16: np.ndarray):
    """Quantize blocks of 32 along the last axis.

    x16: fp16 [..., 32].  Returns (codes uint8 [..., 32] in 0..15, E8M0 scale byte uint8 [...]).
    """
    x = np.asarray(x16, dtype=np.float16)
    assert x.shape[-1] == MX_BLOCK
    amax = np.abs(x.astype(np.float64)).max(axis=-1)
    flat = amax.ravel()
    e = np.array([floor_log2(a) - E2M1_EMAX if a > 0 else -127 for a in flat], dtype=np.int64).reshape(amax.shape)
    sbyte = (e + 127).astype(np.uint8)
    X = np.where(amax > 0, np.ldexp(1.0, e), 0.0)
    codes = e2m1_encode(x, X[..., None])
    return codes, sbyte


def mxfp4_dequantize(codes: np.ndarray, sbyte: np.ndarray) -> np.ndarray:
    return e2m1_decode(codes) * e8m0_decode(sbyte)[..., None]


def quantize_tokens(x16: np.ndarray, fmt: str, tensor: str = "v"):
    """Quantize token rows of head_dim 128: x16 fp16 [N, 128] (tensor "k" or "v": only the
    per-channel formats treat K differently).

    Returns a dict with the stored fields:
      affine: codes [N,128], S [N,128/g], Z [N,128/g] (g the group size)
      per-channel K: codes [N,128], S [N/128, 128], Z [N/128, 128] (one pair per dim and window)
      nvfp4 : codes [N,128], scale [N,8]
      mxfp4 : codes [N,128], scale [N,4] (E8M0 bytes)
      fp8   : codes [N,128] (E4M3 bytes)
      fp16  : codes [N,128] (uint16 fp16 bit patterns)
    """
    x16 = np.asarray(x16, dtype=np.float16)
    N, D = x16.shape
    ap = affine_params(fmt)
    if ap and k_per_channel(fmt) and tensor == "k":
        assert N % KC_WINDOW == 0, "per-channel K is quantized in whole windows"
        w = x16.reshape(N // KC_WINDOW, KC_WINDOW, D).transpose(0, 2, 1)          # [window, dim, token]
        q, S, Z = affine_quantize(w, ap[0])
        return {"codes": np.ascontiguousarray(q.transpose(0, 2, 1)).reshape(N, D), "S": S, "Z": Z}
    if ap:
        nb, gs = ap
        q, S, Z = affine_quantize(x16.reshape(N, D // gs, gs), nb)
        return {"codes": q.reshape(N, D), "S": S, "Z": Z}
    if fmt == "nvfp4":
        c, s = nvfp4_quantize(x16.reshape(N, D // NV_BLOCK, NV_BLOCK))
        return {"codes": c.reshape(N, D), "scale": s}
    if fmt == "mxfp4":
        c, s = mxfp4_quantize(x16.reshape(N, D // MX_BLOCK, MX_BLOCK))
        return {"codes": c.reshape(N, D), "scale": s}
    if fmt == "fp8":
        return {"codes": e4m3_cast(x16)}
    if fmt == "fp16":
        return {"codes": x16.view(np.uint16).copy()}
    raise ValueError(fmt)


def dequantize_tokens(qt: dict, fmt: str, tensor: str = "v") -> np.ndarray:
    """float64 [N, 128] decoded values of quantize_tokens()' output."""
    codes = qt["codes"]
    N, D = codes.shape
    if k_per_channel(fmt) and tensor == "k":
        c = codes.reshape(N // KC_WINDOW, KC_WINDOW, D).transpose(0, 2, 1)
        return affine_dequantize(c, qt["S"], qt["Z"]).transpose(0, 2, 1).reshape(N, D)
    ap = affine_params(fmt)
    if ap:
        gs = ap[1]
        return affine_dequantize(codes.reshape(N, D // gs, gs), qt["S"], qt["Z"]).reshape(N, D)
    if fmt == "nvfp4":
        return nvfp4_dequantize(codes.reshape(N, D // NV_BLOCK, NV_BLOCK), qt["scale"]).reshape(N, D)
    if fmt == "mxfp4":
        return mxfp4_dequantize(codes.reshape(N, D // MX_BLOCK, MX_BLOCK), qt["scale"]).reshape(N, D)
    if fmt == "fp8":
        return e4m3_decode(codes)
    if fmt == "fp16":
        return np.asarray(codes, np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(fmt)
