"""Byte layout of one 128-slot cache block and of the fp16 residual (head_dim 128).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This module packs stored fields into bytes following the written layout
specification, independently of the HIP code that implements the same spec.

Notation: a block holds 128 token slots t = 0..127; D = 128 dims; n = code bits.
"n-bit little-endian field string": field f occupies bits [f*n, f*n + n) of the
byte string, bit b of the string being bit (b mod 8) of byte b // 8.

Affine block (n in {2, 4, 8}), 4096*n + 2048 bytes:
  Kc  @ 0          128 rows (slot t) x 16n bytes; row t = field string of the 128
                   codes of token t, field d = dim d.
  Km  @ 2048n      128 x 8 bytes; slot t: fp16 S0, Z0, S1, Z1 (group 0 = dims 0..63).
  Vc  @ 2048n+1024 128 rows (dim d) x 16n bytes; row d = field string of 128
                   codes, field f holding slot sigma_n(f) (below).
  Vm  @ 4096n+1024 64 entries of 16 bytes, entry (g, q, tau) at ((g*4+q)*8+tau)*16:
                   fp16 S of slots 16tau+4q+i for i = 0..3, then fp16 Z of the same.
NVFP4 block, 18432 bytes:
  Kc  @ 0      128 rows x 64 bytes; 4-bit field d = E2M1 code of dim d.
  Ks  @ 8192   128 rows x 8 bytes; byte b = E4M3 scale of dims 16b..16b+15.
  Vc  @ 9216   128 rows (dim d) x 64 bytes; 4-bit field f holds slot sigma_4(f).
  Vs  @ 17408  8 rows (16-dim block b) x 128 bytes; byte p of row b holds the scale
               of slot rho(p) = 16*((p mod 32) div 4) + 4*(p div 32) + (p mod 4).

sigma_n(f): quarter q = f div 32, k = f mod 32; with F = 32/n fields per 32-bit
word, (j, k') = divmod(k, F), s = k' mod (F/2), hi = k' div (F/2):
    tau = (F/4)*j + 2*(s div 4) + ((s mod 4) div 2),   i = 2*(s mod 2) + hi,
    slot = 16*tau + 4*q + i.
(Each quarter q holds the 32 slots with (slot mod 16) div 4 == q, i.e. the
slots one lane group consumes; inside a 32-bit word the order matches a
two-at-a-time integer-to-fp16 unpack.)

Residual (fp16, per layer and (batch, kv_head)), R slots (R a multiple of 16):
  K @ 0        [R][128] fp16, slot-major.
  V @ 256*R    [R/16][128][16] fp16: slot t, dim d at ((t div 16)*128 + d)*16 + t mod 16.
"""
from __future__ import annotations

import numpy as np

D = 128
BLOCK = 128


def affine_block_bytes(n: int) -> int:
    return 4096 * n + 2048


NVFP4_BLOCK_BYTES = 18432


def block_bytes(fmt: str) -> int:
    if fmt == "nvfp4":
        return NVFP4_BLOCK_BYTES
    return affine_block_bytes(int(fmt[3:]))


def sigma(n: int) -> np.ndarray:
    """sigma_n as an array: field index f (0..127) -> slot."""
    F = 32 // n
    out = np.empty(128, dtype=np.int64)
    for f in range(128):
        q, k = divmod(f, 32)
        j, kp = divmod(k, F)
        s, hi = kp % (F // 2), kp // (F // 2)
        tau = (F // 4) * j + 2 * (s // 4) + ((s % 4) // 2)
        i = 2 * (s % 2) + hi
        out[f] = 16 * tau + 4 * q + i
    return out


def rho() -> np.ndarray:
    p = np.arange(128)
    return 16 * ((p % 32) // 4) + 4 * (p // 32) + (p % 4)


def pack_fields(fields: np.ndarray, n: int) -> np.ndarray:
    """n-bit little-endian field string: fields uint [..., m] -> bytes uint8 [..., m*n/8]."""
    fields = np.asarray(fields, dtype=np.uint64)
    m = fields.shape[-1]
    per = 8 // n
    f = fields.reshape(fields.shape[:-1] + (m // per, per))
    out = np.zeros(f.shape[:-1], dtype=np.uint64)
    for j in range(per):
        out |= (f[..., j] & ((1 << n) - 1)) << np.uint64(j * n)
    return out.astype(np.uint8)


def f16_bytes(a: np.ndarray) -> np.ndarray:
    """fp16 array [..., m] -> little-endian bytes [..., 2m]."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float16))
    return a.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * 2,))


def pack_affine_block(n: int, kq: dict, vq: dict, used: int) -> np.ndarray:
    """One affine block.  kq/vq: quantize_tokens() output for the block's slots
    (arrays of length `used` <= 128); slots >= used are all-zero bytes."""
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    Sk = np.zeros((BLOCK, 2), np.float16); Sk[:used] = kq["S"]
    Zk = np.zeros((BLOCK, 2), np.float16); Zk[:used] = kq["Z"]
    Sv = np.zeros((BLOCK, 2), np.float16); Sv[:used] = vq["S"]
    Zv = np.zeros((BLOCK, 2), np.float16); Zv[:used] = vq["Z"]

    kc = pack_fields(codes_k, n).ravel()                                   # 128 x 16n
    km = f16_bytes(np.stack([Sk[:, 0], Zk[:, 0], Sk[:, 1], Zk[:, 1]], axis=1)).ravel()
    vc = pack_fields(codes_v.T[:, sigma(n)], n).ravel()                    # row d: fields in sigma order
    vm = np.zeros(1024, np.uint8)
    for g in range(2):
        for q in range(4):
            for tau in range(8):
                slots = 16 * tau + 4 * q + np.arange(4)
                e = ((g * 4 + q) * 8 + tau) * 16
                vm[e:e + 8] = f16_bytes(Sv[slots, g])
                vm[e + 8:e + 16] = f16_bytes(Zv[slots, g])
    out = np.concatenate([kc, km, vc, vm])
    assert out.size == affine_block_bytes(n)
    return out


def pack_nvfp4_block(kq: dict, vq: dict, used: int) -> np.ndarray:
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    sk = np.zeros((BLOCK, 8), np.uint8); sk[:used] = kq["scale"]
    sv = np.zeros((BLOCK, 8), np.uint8); sv[:used] = vq["scale"]
    kc = pack_fields(codes_k, 4).ravel()
    ks = sk.ravel()
    vc = pack_fields(codes_v.T[:, sigma(4)], 4).ravel()
    vs = sv.T[:, rho()].ravel()
    out = np.concatenate([kc, ks, vc, vs])
    assert out.size == NVFP4_BLOCK_BYTES
    return out


def pack_arena(fmt: str, kq: dict, vq: dict) -> np.ndarray:
    """Pack N quantized token slots into ceil(N/128) blocks -> uint8 [nblocks, block_bytes]."""
    N = kq["codes"].shape[0]
    nblk = (N + BLOCK - 1) // BLOCK
    blocks = []
    for b in range(nblk):
        lo, hi = b * BLOCK, min(N, (b + 1) * BLOCK)
        sl = {k: v[lo:hi] for k, v in kq.items()}
        sv = {k: v[lo:hi] for k, v in vq.items()}
        if fmt == "nvfp4":
            blocks.append(pack_nvfp4_block(sl, sv, hi - lo))
        else:
            blocks.append(pack_affine_block(int(fmt[3:]), sl, sv, hi - lo))
    if not blocks:
        return np.zeros((0, block_bytes(fmt)), np.uint8)
    return np.stack(blocks)


def residual_bytes(R: int) -> int:
    return 512 * R


def pack_residual(k16: np.ndarray, v16: np.ndarray, R: int) -> tuple[np.ndarray, np.ndarray]:
    """Residual layout for r = len(k16) <= R slots.  Returns (bytes [512R], valid-mask [512R])
    so that callers compare only bytes of occupied slots."""
    r = k16.shape[0]
    K = np.zeros((R, D), np.float16); K[:r] = k16
    V = np.zeros((R, D), np.float16); V[:r] = v16
    kmask = np.zeros((R, D), bool); kmask[:r] = True
    Vt = V.reshape(R // 16, 16, D).transpose(0, 2, 1)           # [tile][d][slot in tile]
    vmask = kmask.reshape(R // 16, 16, D).transpose(0, 2, 1)
    data = np.concatenate([f16_bytes(K.ravel()), f16_bytes(np.ascontiguousarray(Vt).ravel())])
    mask = np.concatenate([np.repeat(kmask.ravel(), 2), np.repeat(np.ascontiguousarray(vmask).ravel(), 2)])
    return data, mask
