"""Pins of the oracle's block packer against hand-derived byte positions and structural properties."""
import json
import os

import numpy as np
import pytest

from oracle import layout, quant

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_cases.json")))


def _ng(fmt):
    ap = quant.affine_params(fmt)
    return 128 // ap[1] if ap else 0


def _empty(fmt):
    if fmt == "fp16":
        return {"codes": np.zeros((128, 128), np.uint16)}
    if fmt == "fp8":
        return {"codes": np.zeros((128, 128), np.uint8)}
    if fmt == "nvfp4":
        return {"codes": np.zeros((128, 128), np.uint8), "scale": np.zeros((128, 8), np.uint8)}
    if fmt == "mxfp4":
        return {"codes": np.zeros((128, 128), np.uint8), "scale": np.zeros((128, 4), np.uint8)}
    return {"codes": np.zeros((128, 128), np.uint8), "S": np.zeros((128, _ng(fmt)), np.float16),
            "Z": np.zeros((128, _ng(fmt)), np.float16)}


def _pack(fmt, kq, vq):
    if fmt == "fp16":
        return layout.pack_fp16_block(kq, vq, 128)
    if fmt == "fp8":
        return layout.pack_fp8_block(kq, vq, 128)
    if fmt == "nvfp4":
        return layout.pack_nvfp4_block(kq, vq, 128)
    if fmt == "mxfp4":
        return layout.pack_mxfp4_block(kq, vq, 128)
    n, gs = quant.affine_params(fmt)
    return layout.pack_affine_block(n, kq, vq, 128, gs)


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: f"{c['fmt']}-{c['part']}-{c['slot']}-{c['dim']}")
def test_code_positions(case):
    kq, vq = _empty(case["fmt"]), _empty(case["fmt"])
    (kq if case["part"] == "Kc" else vq)["codes"][case["slot"], case["dim"]] = case["code"]
    blk = _pack(case["fmt"], kq, vq)
    nz = np.flatnonzero(blk)
    assert list(nz) == [case["byte"]]
    assert blk[case["byte"]] == (case["code"] << case["shift"]) & 0xFF


@pytest.mark.parametrize("case", GOLDEN["meta_cases"], ids=lambda c: f"{c['fmt']}-{c['part']}-{c['slot']}-{c['field']}")
def test_meta_positions(case):
    kq, vq = _empty(case["fmt"]), _empty(case["fmt"])
    (kq if case["part"] == "Km" else vq)[case["field"]][case["slot"], case["group"]] = 1.5   # 0x3E00
    blk = _pack(case["fmt"], kq, vq)
    assert list(np.flatnonzero(blk)) == [case["byte"] + 1]
    assert blk[case["byte"] + 1] == 0x3E


@pytest.mark.parametrize("case", GOLDEN["scale_cases"], ids=lambda c: f"{c['part']}-{c['slot']}")
def test_scale_positions(case):
    kq, vq = _empty("nvfp4"), _empty("nvfp4")
    (kq if case["part"] == "Ks" else vq)["scale"][case["slot"], case["dim"] // 16] = 0x38
    blk = _pack("nvfp4", kq, vq)
    assert list(np.flatnonzero(blk)) == [case["byte"]]


@pytest.mark.parametrize("case", GOLDEN["mx_scale_cases"], ids=lambda c: f"{c['part']}-{c['slot']}")
def test_mx_scale_positions(case):
    kq, vq = _empty("mxfp4"), _empty("mxfp4")
    (kq if case["part"] == "Ks" else vq)["scale"][case["slot"], case["dim"] // 32] = 0x7F
    blk = _pack("mxfp4", kq, vq)
    assert list(np.flatnonzero(blk)) == [case["byte"]]


@pytest.mark.parametrize("case", GOLDEN["kc_meta_cases"], ids=lambda c: f"{c['fmt']}-{c['field']}-{c['dim']}")
def test_per_channel_k_meta_positions(case):
    n = quant.affine_params(case["fmt"])[0]
    kq = {"codes": np.zeros((128, 128), np.uint8), "S": np.zeros(128, np.float16), "Z": np.zeros(128, np.float16)}
    kq[case["field"]][case["dim"]] = 1.5                                   # 0x3E00
    blk = layout.pack_affine_kc_block(n, kq, _empty("int4"))
    assert list(np.flatnonzero(blk)) == [case["byte"] + 1] and blk[case["byte"] + 1] == 0x3E


@pytest.mark.parametrize("n", [2, 4, 8])
def test_per_channel_k_block_coverage(n):
    """All-ones codes, S, Z and V fields fill the whole block; the operand order lists every
    dim once per block and each quarter's 32 dims are the quarter's K lane dims."""
    ones = np.uint16(0xFFFF).view(np.float16)
    kq = {"codes": np.full((128, 128), (1 << n) - 1, np.uint8), "S": np.full(128, ones), "Z": np.full(128, ones)}
    vq = {"codes": np.full((128, 128), (1 << n) - 1, np.uint8), "S": np.full((128, 2), ones), "Z": np.full((128, 2), ones)}
    blk = layout.pack_affine_kc_block(n, kq, vq)
    assert np.all(blk == 0xFF) and blk.size == layout.block_bytes(f"int{n}kc") == 4096 * n + 1536
    order = [layout.k_operand_dims(n, g) for g in range(4)]
    assert sorted(np.concatenate([o.ravel() for o in order])) == list(range(128))
    for g in range(4):
        assert sorted(order[g].ravel()) == sorted(layout.k_lane_dims(f"int{n}", g))


@pytest.mark.parametrize("case", GOLDEN["residual_cases"], ids=lambda c: c["part"])
def test_residual_positions(case):
    R = case["R"]
    k = np.zeros((R, 128), np.float16); v = np.zeros((R, 128), np.float16)
    (k if case["part"] == "K" else v)[case["slot"], case["dim"]] = 1.5
    data, mask = layout.pack_residual(k, v, R)
    assert list(np.flatnonzero(data)) == [case["byte"] + 1]


@pytest.mark.parametrize("fmt", ["int2", "int4", "int8", "int2g32", "int4g32", "int8g32", "int4g128",
                                 "nvfp4", "mxfp4", "fp8", "fp16"])
def test_v_lane_fields_cover_every_slot_and_dim_once(fmt):
    """Every (slot, dim) of the block is held by exactly one (part, lane, field), and each
    lane's 8 operand positions e are the slots 16(e div 4) + 4g + (e mod 4) of its part."""
    k, e = layout.v_lane_fields(fmt)
    seen = np.zeros((128, 128), np.int64)
    for w in range(4):
        for L in range(64):
            g, c = L // 16, L % 16
            seen[layout.lane_slot(w, g, e), 16 * k + c] += 1
    assert np.all(seen == 1)
    # each dim tile k gets all 8 positions once
    for kk in range(8):
        assert sorted(e[k == kk]) == list(range(8))


@pytest.mark.parametrize("fmt", ["int2", "int4", "int8", "int2g32", "int4g32", "int8g32", "int4g128",
                                 "nvfp4", "mxfp4", "fp8", "fp16"])
def test_k_lane_dims_cover_every_dim_once_per_slot(fmt):
    """The four lane quarters of a slot hold all 128 dims once; in affine formats each
    16-field half of a lane lies in one 64-dim group."""
    d = np.concatenate([layout.k_lane_dims(fmt, g) for g in range(4)])
    assert sorted(d) == list(range(128))
    ap = quant.affine_params(fmt)
    if ap and ap[1] != 32:
        f = np.arange(32)
        for g in range(4):
            assert np.all(layout.k_lane_dims(fmt, g) // 64 == f // 16)
    if ap and ap[1] == 32:
        # quarter g holds the dims 32j + 8g .. 32j + 8g + 7 of every 32-dim group j
        for g in range(4):
            assert np.all((layout.k_lane_dims(fmt, g) % 32) // 8 == g)


def test_every_bit_of_a_block_is_reachable_once():
    """Setting all codes/meta to all-ones fills every byte of the block with 0xFF
    (no gaps, and codes of different elements never share bits)."""
    for fmt in ("int2", "int4", "int8", "int2g32", "int4g32", "int8g32", "int2g128", "int4g128", "int8g128"):
        n, gs = quant.affine_params(fmt)
        full = {"codes": np.full((128, 128), (1 << n) - 1, np.uint8),
                "S": np.full((128, 128 // gs), np.uint16(0xFFFF).view(np.float16)),
                "Z": np.full((128, 128 // gs), np.uint16(0xFFFF).view(np.float16))}
        blk = layout.pack_affine_block(n, full, full, 128, gs)
        assert np.all(blk == 0xFF) and blk.size == layout.affine_block_bytes(n, gs)
    full = {"codes": np.full((128, 128), 15, np.uint8), "scale": np.full((128, 8), 0xFF, np.uint8)}
    blk = layout.pack_nvfp4_block(full, full, 128)
    assert np.all(blk == 0xFF) and blk.size == layout.NVFP4_BLOCK_BYTES
    full = {"codes": np.full((128, 128), 15, np.uint8), "scale": np.full((128, 4), 0xFF, np.uint8)}
    blk = layout.pack_mxfp4_block(full, full, 128)
    assert np.all(blk == 0xFF) and blk.size == layout.MXFP4_BLOCK_BYTES
    full = {"codes": np.full((128, 128), 0xFF, np.uint8)}
    blk = layout.pack_fp8_block(full, full, 128)
    assert np.all(blk == 0xFF) and blk.size == layout.FP8_BLOCK_BYTES
    full = {"codes": np.full((128, 128), 0xFFFF, np.uint16)}
    blk = layout.pack_fp16_block(full, full, 128)
    assert np.all(blk == 0xFF) and blk.size == layout.FP16_BLOCK_BYTES


def test_fp16_block_holds_every_value_once():
    """Distinct bit patterns in every (slot, dim) of K and V: the block is a permutation of
    the 2 x 16384 values (each at an even byte offset, low byte first)."""
    k = (np.arange(128 * 128, dtype=np.uint32).reshape(128, 128) * 2 + 1).astype(np.uint16)
    v = (np.arange(128 * 128, dtype=np.uint32).reshape(128, 128) * 2).astype(np.uint16)
    blk = layout.pack_fp16_block({"codes": k}, {"codes": v}, 128)
    vals = blk.view("<u2")
    assert sorted(vals[:16384]) == sorted(k.ravel())
    assert sorted(vals[16384:]) == sorted(v.ravel())


def test_partial_block_tail_is_zero():
    full = {"codes": np.full((128, 128), 3, np.uint8), "S": np.ones((128, 2), np.float16),
            "Z": np.ones((128, 2), np.float16)}
    used = 37
    part = {k: v[:used] for k, v in full.items()}
    blk = layout.pack_affine_block(2, part, part, used)
    ref = layout.pack_affine_block(2, {k: np.where(np.arange(128)[:, None] < used, v, 0).astype(v.dtype)
                                       for k, v in full.items()},
                                   {k: np.where(np.arange(128)[:, None] < used, v, 0).astype(v.dtype)
                                    for k, v in full.items()}, 128)
    assert np.array_equal(blk, ref)
