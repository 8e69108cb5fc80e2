"""Byte layout of one 128-slot cache block and of the fp16 residual (head_dim 128).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This module packs stored fields into bytes following the written layout
specification, independently of the HIP code that implements the same spec.
The pages fix no byte layout (only that codes are stored as n-bit integers with
S and Z per group, page "KV缓存量化技术：提升大模型长文本生成效率" §2.1, and that NVFP4
stores E2M1 codes with one FP8 scale per 16 values, page "NVFP4 KV缓存技术详解" §2.1);
the layout below is this cache's own.

Notation: a block holds 128 token slots t = 0..127; D = 128 dims; n = code bits
(NVFP4 codes are 4-bit fields).  "n-bit little-endian field string": field f
occupies bits [f*n, f*n + n) of the byte string, bit b of the string being bit
(b mod 8) of byte b // 8.  A block is [Kc][Km][Vc][Vm].

Kc (2048n bytes; NVFP4 8192): 4 parts w x 2 tiles u x 64 lanes L (g = L div 16,
    c = L mod 16), each lane holding 4n bytes (NVFP4 16) of slot t = 32w + 16u + c:
    the field string of 32 fields, field f holding the code of dim
    64(f div 16) + 16g + (f mod 16) (affine, groups of 64 or 128) or of dim 32g + f (NVFP4).
    Affine groups of 32: field f holds dim 32j + 8g + e, where (j, e) is f's place among the
    decode kernel's MFMA operands (step j, element e; every step then covers one group):
      INT4: j = f div 8, r = f mod 8, e = 2(r mod 4) + r div 4
      INT8: j = f div 8, r = f mod 8, e = 4(r div 4) + 2(r mod 2) + (r div 2) mod 2
      INT2: j = 2(f div 16) + (f div 4) mod 2, r = f mod 16, e = 2(r mod 4) + r div 8  Lane data
    is stored in chunks of min(16, 4n) bytes: chunk r of lane L of (w, u) at
    (((2w + u)*K + r)*64 + L)*min(16, 4n), K = 4n / min(16, 4n) (INT2 8-byte
    chunks, INT4 and NVFP4 one 16-byte chunk, INT8 two 16-byte chunks).
Km, affine (512 NG bytes, NG = 128/g groups per token): 8 tiles tau of 64 NG bytes (slots
    16tau + r, r = 0..15): fp16 S of group G at tau*64NG + 2(NG r + G), fp16 Z at
    tau*64NG + 32NG + 2(NG r + G) (NG = 2: S at tau*128 + 4r + 2G, Z 64 bytes later).
Km, NVFP4 (1024 bytes): 2 bytes per (w, u, L) at ((2w + u)*64 + L)*2: the E4M3
    scales of dims 32g..32g+15 and 32g+16..32g+31 of slot 32w + 16u + c.
Vc (2048n bytes; NVFP4 8192): 4 parts w, each 64 lanes L (g = L div 16,
    c = L mod 16) of 8n bytes, stored as n/2 chunks of 16 bytes: chunk r of lane
    L of part w at ((w*(n/2) + r)*64 + L)*16.  The lane's 8n bytes are the field
    string of 64 fields phi; field phi holds the code of dim 16k + c and slot
    32w + 16(e div 4) + 4g + (e mod 4), with (k, e) given by:
      INT4:  k = phi div 8, v = phi mod 8, e = 2(v mod 4) + v div 4
      NVFP4: k = phi div 8, e = phi mod 8
      INT2:  u = phi div 16, m = phi mod 16, k = 2u + (m div 4) mod 2,
             e = 2(m mod 4) + m div 8
      INT8:  u = phi div 4, b = phi mod 4, k = u div 2,
             e = 4(u mod 2) + 2(b mod 2) + b div 2
Per-channel K ("int{n}kc"): Kc as groups of 64; Km (512 bytes) holds the block's per-dim S
    (256 bytes) then Z: fp16 at 2(32g + 8j + e) for the dim fed by element e of MFMA k-step j
    in lane quarter g (the dim of the field f whose (j, e) is that pair, in the table above);
    Vc and Vm as groups of 64.
Vm, affine (512 NG bytes): 8 tiles tau x 4 quarters g of 16 NG bytes at (4tau + g)*16NG:
    fp16 S of group G for slots 16tau + 4g + i (i = 0..3) at 8G + 2i, then the Z likewise
    from 8NG (NG = 2: S of group 0, S of group 1, Z of group 0, Z of group 1).
Vm, NVFP4 (1024 bytes): byte ((4w + g)*8 + k)*8 + e = E4M3 scale of dims
    16k..16k+15 of slot 32w + 16(e div 4) + 4g + (e mod 4).

MXFP4 block (17408 bytes): [Kc][Ks][Vc][Vs].
Kc (8192 bytes): as NVFP4's (lane quarter g of a slot holds dims 32g .. 32g+31: one MX block).
Ks (512 bytes): byte ((2w + u)*64 + L) = E8M0 scale of that lane's block (slot 32w + 16u + c,
    dims 32g .. 32g+31).
Vc (8192 bytes): the chunk scheme of NVFP4's Vc with field phi holding k = 2(phi div 16) +
    (phi mod 2), e = (phi div 2) mod 8: byte 8m + e of a lane string holds slot e's values at
    dims 16(2m) + c (low nibble) and 16(2m+1) + c (high nibble), two dims of one MX block.
Vs (512 bytes): byte ((4w + g)*4 + m)*8 + e = E8M0 scale of dims 32m .. 32m+31 of slot
    32w + 16(e div 4) + 4g + (e mod 4).

FP8 block (32768 bytes): [Kc][Vc], the Kc and Vc regions of INT8 (n = 8) with E4M3 bytes as
the codes, Vc at 16384; no metadata (the scale is fixed).

FP16 block (65536 bytes): [Kc][Vc] with n = 16 (every field an fp16 value, little-endian) and
the fields in NVFP4's order: Kc lane field f of quarter g holds dim 32g + f (4 chunks of 16
bytes per lane); Vc field phi has k = phi div 8, e = phi mod 8 (8 chunks per lane), Vc at
32768; no metadata.

Residual (fp16, per layer and (batch, kv_head)), R slots (R a multiple of 16):
  K @ 0        [R][128] fp16, slot-major.
  V @ 256*R    [R/16][128][16] fp16: slot t, dim d at ((t div 16)*128 + d)*16 + t mod 16.
"""
from __future__ import annotations

import numpy as np

from .quant import affine_params, k_per_channel

D = 128
BLOCK = 128


def affine_block_bytes(n: int, gs: int = 64, kc: bool = False) -> int:
    if kc:
        return 4096 * n + 512 + 1024
    return 4096 * n + 1024 * (128 // gs)


NVFP4_BLOCK_BYTES = 18432
MXFP4_BLOCK_BYTES = 17408
FP8_BLOCK_BYTES = 32768
FP16_BLOCK_BYTES = 65536


def block_bytes(fmt: str) -> int:
    if fmt == "nvfp4":
        return NVFP4_BLOCK_BYTES
    if fmt == "mxfp4":
        return MXFP4_BLOCK_BYTES
    if fmt == "fp8":
        return FP8_BLOCK_BYTES
    if fmt == "fp16":
        return FP16_BLOCK_BYTES
    n, gs = affine_params(fmt)
    return affine_block_bytes(n, gs, k_per_channel(fmt))


def k_lane_dims(fmt: str, g: int) -> np.ndarray:
    """Kc lane field string of lane quarter g: field f (0..31) -> dim."""
    f = np.arange(32)
    if fmt in ("nvfp4", "mxfp4", "fp16"):
        return 32 * g + f
    ap = affine_params(fmt)
    if ap and ap[1] == 32:
        j, e = step_elem(ap[0], f)
        return 32 * j + 8 * g + e
    return 64 * (f // 16) + 16 * g + f % 16


def step_elem(n: int, f):
    """(k-step j, element e) of the decode kernel's MFMA operand that K lane field f feeds."""
    f = np.asarray(f)
    if n == 2:
        j, r = 2 * (f // 16) + (f // 4) % 2, f % 16
        e = 2 * (r % 4) + r // 8
    elif n == 4:
        j, r = f // 8, f % 8
        e = 2 * (r % 4) + r // 4
    else:
        j, r = f // 8, f % 8
        e = 4 * (r // 4) + 2 * (r % 2) + (r // 2) % 2
    return j, e


def k_operand_dims(n: int, g: int) -> np.ndarray:
    """[4, 8]: dim fed by element e of k-step j in lane quarter g (K lanes of groups of 64)."""
    f = np.arange(32)
    j, e = step_elem(n, f)
    out = np.full((4, 8), -1, np.int64)
    out[j, e] = k_lane_dims(f"int{n}", g)
    return out


def _pack_kc(fmt: str, codes_k: np.ndarray) -> np.ndarray:
    """Kc region from the [slot, dim] code array."""
    n = code_bits(fmt)
    lane_bytes = 4 * n
    cb = min(16, lane_bytes)
    K = lane_bytes // cb
    out = np.zeros((4, 2, K, 64, cb), np.uint8)
    for w in range(4):
        for u in range(2):
            for L in range(64):
                g, c = L // 16, L % 16
                t = 32 * w + 16 * u + c
                out[w, u, :, L, :] = pack_fields(codes_k[t, k_lane_dims(fmt, g)], n).reshape(K, cb)
    return out.ravel()


def v_lane_fields(fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """Vc lane field string: field phi (0..63) -> (dim tile k, operand position e)."""
    phi = np.arange(64)
    if fmt in ("nvfp4", "fp16") or (affine_params(fmt) or (0,))[0] == 4:
        k, v = phi // 8, phi % 8
        e = v if fmt in ("nvfp4", "fp16") else 2 * (v % 4) + v // 4
    elif fmt == "mxfp4":
        k = 2 * (phi // 16) + phi % 2
        e = (phi // 2) % 8
    elif (affine_params(fmt) or (0,))[0] == 2:
        u, m = phi // 16, phi % 16
        k = 2 * u + (m // 4) % 2
        e = 2 * (m % 4) + m // 8
    elif fmt == "fp8" or (affine_params(fmt) or (0,))[0] == 8:
        u, b = phi // 4, phi % 4
        k = u // 2
        e = 4 * (u % 2) + 2 * (b % 2) + b // 2
    else:
        raise ValueError(fmt)
    return k, e


def lane_slot(w: int, g: int, e) -> np.ndarray:
    """Slot of operand position e of a lane in quarter g of part w."""
    e = np.asarray(e)
    return 32 * w + 16 * (e // 4) + 4 * g + (e % 4)


def code_bits(fmt: str) -> int:
    return {"nvfp4": 4, "mxfp4": 4, "fp8": 8, "fp16": 16}.get(fmt) or affine_params(fmt)[0]


def pack_fields(fields: np.ndarray, n: int) -> np.ndarray:
    """n-bit little-endian field string: fields uint [..., m] -> bytes uint8 [..., m*n/8]."""
    if n == 16:
        return np.ascontiguousarray(np.asarray(fields).astype("<u2")).view(np.uint8).reshape(
            np.shape(fields)[:-1] + (2 * np.shape(fields)[-1],))
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


def _pack_vc(fmt: str, codes_v: np.ndarray) -> np.ndarray:
    """Vc region from the [slot, dim] code array."""
    n = code_bits(fmt)
    k, e = v_lane_fields(fmt)
    nchunk = n // 2
    out = np.zeros((4, nchunk, 64, 16), np.uint8)
    for w in range(4):
        for L in range(64):
            g, c = L // 16, L % 16
            fields = codes_v[lane_slot(w, g, e), 16 * k + c]
            out[w, :, L, :] = pack_fields(fields, n).reshape(nchunk, 16)
    return out.ravel()


def pack_affine_block(n: int, kq: dict, vq: dict, used: int, gs: int = 64) -> np.ndarray:
    """One affine block with groups of gs values.  kq/vq: quantize_tokens() output for the
    block's slots (arrays of length `used` <= 128); slots >= used are all-zero bytes."""
    fmt = f"int{n}" if gs == 64 else f"int{n}g{gs}"
    ng = D // gs
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    Sk = np.zeros((BLOCK, ng), np.float16); Sk[:used] = kq["S"]
    Zk = np.zeros((BLOCK, ng), np.float16); Zk[:used] = kq["Z"]
    Sv = np.zeros((BLOCK, ng), np.float16); Sv[:used] = vq["S"]
    Zv = np.zeros((BLOCK, ng), np.float16); Zv[:used] = vq["Z"]

    kc = _pack_kc(fmt, codes_k)
    # per tile: S of (slot r, group G) in order NG r + G, then the Z likewise
    km = np.concatenate([np.concatenate([f16_bytes(Sk[16 * t:16 * t + 16].ravel()),
                                         f16_bytes(Zk[16 * t:16 * t + 16].ravel())]) for t in range(8)])
    vc = _pack_vc(fmt, codes_v)
    vm = np.zeros(512 * ng, np.uint8)
    for t in range(8):
        for g in range(4):
            slots = 16 * t + 4 * g + np.arange(4)
            base = (4 * t + g) * 16 * ng
            for G in range(ng):
                vm[base + 8 * G:base + 8 * G + 8] = f16_bytes(Sv[slots, G])
                vm[base + 8 * ng + 8 * G:base + 8 * ng + 8 * G + 8] = f16_bytes(Zv[slots, G])
    out = np.concatenate([kc, km, vc, vm])
    assert out.size == affine_block_bytes(n, gs)
    return out


def pack_affine_kc_block(n: int, kq: dict, vq: dict) -> np.ndarray:
    """One block of per-channel K (kq: codes [128, 128], S and Z [128] of the block's window)
    and per-token V in groups of 64 (vq as quantize_tokens() gives it for the 128 slots)."""
    fmt = f"int{n}"
    kc = _pack_kc(fmt, np.asarray(kq["codes"], np.uint8))
    order = np.concatenate([k_operand_dims(n, g).ravel() for g in range(4)])    # position -> dim
    km = np.concatenate([f16_bytes(np.asarray(kq["S"], np.float16)[order]),
                         f16_bytes(np.asarray(kq["Z"], np.float16)[order])])
    full = pack_affine_block(n, {"codes": np.zeros((BLOCK, D), np.uint8), "S": np.zeros((BLOCK, 2), np.float16),
                                 "Z": np.zeros((BLOCK, 2), np.float16)}, vq, BLOCK, 64)
    vpart = full[2048 * n + 1024:]                                              # Vc and Vm of groups of 64
    out = np.concatenate([kc, km, vpart])
    assert out.size == affine_block_bytes(n, 64, True)
    return out


def pack_nvfp4_block(kq: dict, vq: dict, used: int) -> np.ndarray:
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    sk = np.zeros((BLOCK, 8), np.uint8); sk[:used] = kq["scale"]
    sv = np.zeros((BLOCK, 8), np.uint8); sv[:used] = vq["scale"]
    kc = _pack_kc("nvfp4", codes_k)
    ks = np.zeros((4, 2, 64, 2), np.uint8)
    for w in range(4):
        for u in range(2):
            for L in range(64):
                g, c = L // 16, L % 16
                ks[w, u, L] = sk[32 * w + 16 * u + c, 2 * g:2 * g + 2]
    ks = ks.ravel()
    vc = _pack_vc("nvfp4", codes_v)
    vs = np.zeros((4, 4, 8, 8), np.uint8)                                   # [w][g][k][e]
    e = np.arange(8)
    for w in range(4):
        for g in range(4):
            vs[w, g] = sv[lane_slot(w, g, e)].T                             # [k][e]
    out = np.concatenate([kc, ks, vc, vs.ravel()])
    assert out.size == NVFP4_BLOCK_BYTES
    return out


def pack_mxfp4_block(kq: dict, vq: dict, used: int) -> np.ndarray:
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    sk = np.zeros((BLOCK, 4), np.uint8); sk[:used] = kq["scale"]
    sv = np.zeros((BLOCK, 4), np.uint8); sv[:used] = vq["scale"]
    kc = _pack_kc("mxfp4", codes_k)
    ks = np.zeros((4, 2, 64), np.uint8)
    for w in range(4):
        for u in range(2):
            for L in range(64):
                ks[w, u, L] = sk[32 * w + 16 * u + L % 16, L // 16]
    vc = _pack_vc("mxfp4", codes_v)
    vs = np.zeros((4, 4, 4, 8), np.uint8)                                   # [w][g][m][e]
    e = np.arange(8)
    for w in range(4):
        for g in range(4):
            vs[w, g] = sv[lane_slot(w, g, e)].T                             # [m][e]
    out = np.concatenate([kc, ks.ravel(), vc, vs.ravel()])
    assert out.size == MXFP4_BLOCK_BYTES
    return out


def pack_fp8_block(kq: dict, vq: dict, used: int) -> np.ndarray:
    codes_k = np.zeros((BLOCK, D), np.uint8); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint8); codes_v[:used] = vq["codes"]
    out = np.concatenate([_pack_kc("fp8", codes_k), _pack_vc("fp8", codes_v)])
    assert out.size == FP8_BLOCK_BYTES
    return out


def pack_fp16_block(kq: dict, vq: dict, used: int) -> np.ndarray:
    codes_k = np.zeros((BLOCK, D), np.uint16); codes_k[:used] = kq["codes"]
    codes_v = np.zeros((BLOCK, D), np.uint16); codes_v[:used] = vq["codes"]
    out = np.concatenate([_pack_kc("fp16", codes_k), _pack_vc("fp16", codes_v)])
    assert out.size == FP16_BLOCK_BYTES
    return out


def pack_arena(fmt: str, kq: dict, vq: dict) -> np.ndarray:
    """Pack N quantized token slots into ceil(N/128) blocks -> uint8 [nblocks, block_bytes]."""
    N = kq["codes"].shape[0]
    nblk = (N + BLOCK - 1) // BLOCK
    blocks = []
    if k_per_channel(fmt):
        n = affine_params(fmt)[0]
        for b in range(nblk):
            sl = slice(b * BLOCK, (b + 1) * BLOCK)
            blocks.append(pack_affine_kc_block(n, {"codes": kq["codes"][sl], "S": kq["S"][b], "Z": kq["Z"][b]},
                                               {k: v[sl] for k, v in vq.items()}))
        return np.stack(blocks) if blocks else np.zeros((0, block_bytes(fmt)), np.uint8)
    for b in range(nblk):
        lo, hi = b * BLOCK, min(N, (b + 1) * BLOCK)
        sl = {k: v[lo:hi] for k, v in kq.items()}
        sv = {k: v[lo:hi] for k, v in vq.items()}
        if fmt == "nvfp4":
            blocks.append(pack_nvfp4_block(sl, sv, hi - lo))
        elif fmt == "mxfp4":
            blocks.append(pack_mxfp4_block(sl, sv, hi - lo))
        elif fmt == "fp8":
            blocks.append(pack_fp8_block(sl, sv, hi - lo))
        elif fmt == "fp16":
            blocks.append(pack_fp16_block(sl, sv, hi - lo))
        else:
            n, gs = affine_params(fmt)
            blocks.append(pack_affine_block(n, sl, sv, hi - lo, gs))
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
