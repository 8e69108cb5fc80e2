"""Number formats used by the cache, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* fp16: IEEE binary16.  `f16()` rounds a float64 once to the nearest binary16,
  ties to even (numpy's double->half conversion; pinned against exact rational
  rounding in the tests).
* E4M3: the OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa bits,
  no infinities, 0x7F/0xFF = NaN, largest finite 448.  Page
  "NVFP4 KV缓存技术详解" (glsqs.com/news/814573) §2.1 says that each group of 16
  values shares one FP8 scale; the scale format is read as E4M3.  The same format
  stores whole FP8 caches (page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存",
  section on the KV cache formats: an FP8 cast with a fixed scale), read as a cast of each
  value with scale 1, saturating at 448.
* E2M1: the 4-bit float of NVFP4 (1 sign, 2 exponent, 1 mantissa bit), with
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E8M0: the power-of-two scale of the microscaling (MX) formats, byte b = 2^(b - 127),
  0xFF = NaN; page "NVFP4 KV缓存技术详解" §3.2 compares NVFP4 with MXFP4 (E2M1 elements
  sharing one such scale per 32 values).
"""
from __future__ import annotations

import math
import numpy as np

F16_MAX = 65504.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def f16(x) -> np.ndarray:
    """Round float64 values once to binary16, ties to even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def f16_saturate(x) -> np.ndarray:
    """Round to binary16 after clamping to the finite range [-65504, 65504]; -0 becomes +0."""
    x = np.clip(np.asarray(x, dtype=np.float64), -F16_MAX, F16_MAX)
    return f16(x + 0.0)


# ----------------------------------------------------------------------------- E4M3

def e4m3_decode(code) -> np.ndarray:
    """Value of E4M3 bytes as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def _rne(x: float) -> int:
    """Round a float to the nearest integer, ties to even (Python's round())."""
    return int(round(x))


def e4m3_encode_scalar(v: float) -> int:
    """Non-negative float -> E4M3 byte: round to nearest, ties to even mantissa, saturate at 448.

    Works on the binade of v: below 2**-6 the grid is the subnormal step 2**-9;
    inside binade [2**e, 2**(e+1)) the grid step is 2**(e-3).
    """
    if not v >= 0.0:
        raise ValueError("E4M3 scale must be non-negative and not NaN")
    if v >= E4M3_MAX:
        return E4M3_MAX_CODE
    if v < 2.0 ** -6:
        k = _rne(v * 2.0 ** 9)          # 0..8; 8 is the smallest normal (code 0x08)
        return k
    e = math.floor(math.log2(v))
    # guard against log2 rounding at exact powers of two
    if 2.0 ** e > v:
        e -= 1
    elif 2.0 ** (e + 1) <= v:
        e += 1
    k = _rne((v / 2.0 ** e - 1.0) * 8.0)  # 0..8
    if k == 8:
        e, k = e + 1, 0
    code = ((e + 7) << 3) | k
    return min(code, E4M3_MAX_CODE)


def e4m3_encode(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    out = np.fromiter((e4m3_encode_scalar(float(x)) for x in v.ravel()), dtype=np.uint8, count=v.size)
    return out.reshape(v.shape)


_E4M3_CAST_TABLE = None


def _e4m3_cast_table() -> np.ndarray:
    """Signed E4M3 byte of every fp16 bit pattern (finite ones; inf/NaN patterns map to the
    saturated code of their sign), from e4m3_encode_scalar on the magnitude."""
    global _E4M3_CAST_TABLE
    if _E4M3_CAST_TABLE is None:
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        mag = np.abs(bits.view(np.float16).astype(np.float64))
        mag = np.where(np.isfinite(mag), mag, E4M3_MAX)
        table = np.array([e4m3_encode_scalar(float(m)) for m in mag], dtype=np.uint8)
        table |= np.where(bits & 0x8000, 0x80, 0).astype(np.uint8)
        _E4M3_CAST_TABLE = table
    return _E4M3_CAST_TABLE


def e4m3_cast(x16) -> np.ndarray:
    """fp16 values -> E4M3 bytes: magnitude rounded to nearest, ties to even mantissa,
    saturating at 448; the sign bit is kept (so -0 and negatives that round to 0 give 0x80)."""
    x = np.ascontiguousarray(np.asarray(x16, dtype=np.float16))
    return _e4m3_cast_table()[x.view(np.uint16)]


# ----------------------------------------------------------------------------- E2M1

# Midpoints between consecutive E2M1 magnitudes.
_E2M1_MIDPOINTS = np.array([(a + b) / 2 for a, b in zip(E2M1_MAGNITUDES[:-1], E2M1_MAGNITUDES[1:])])


def e2m1_encode(x16: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Signed E2M1 codes of fp16 values x against a positive-or-zero scale s (broadcast).

    magnitude index = nearest grid point of min(|x|/s, 6), ties to the even index,
    decided by comparing |x| with midpoint*s (both exact in float64).
    sign bit = sign bit of x (so -0 and negatives that round to 0 give 0x8).
    s == 0 gives signed zeros.
    """
    x = np.asarray(x16, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    a = np.abs(x)
    thr = _E2M1_MIDPOINTS * s[..., None]                       # [..., 7]
    below = (a[..., None] > thr).sum(axis=-1)                  # midpoints strictly below |x|
    tie = (a[..., None] == thr)
    k_tie = np.argmax(tie, axis=-1)
    idx = np.where(tie.any(axis=-1), np.where(k_tie % 2 == 0, k_tie, k_tie + 1), below)
    idx = np.where(s == 0, 0, idx)
    sign = np.signbit(x).astype(np.int64) * 8
    return (idx + sign).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDES)[c & 7]
    return np.where(c & 8, -mag, mag)


def e8m0_decode(byte) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - 127))


def floor_log2(a: float) -> int:
    """floor(log2(a)) of a positive finite float, exactly (frexp: a = m 2^e, 0.5 <= m < 1)."""
    m, e = math.frexp(a)
    return e - 1
