"""Pins of the size formula against the pages' tables."""
import json
import os

import pytest

from oracle import sizes

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_size_tables.json")))
GiB = 2 ** 30


def test_p2_savings_table():
    t = G["p2_savings"]; m = t["model"]
    for row in t["rows"]:
        for fmt, bpv in (("fp16", 2), ("fp8", 1), ("nvfp4", 0.5)):
            got = sizes.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], row["tokens"], bpv)
            assert got == row[fmt] * GiB
    fp16 = sizes.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], 131072, 2)
    fp8 = sizes.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], 131072, 1)
    assert 8 * (fp16 - fp8) == t["fp8_saving_128k_x8_GiB"] * GiB


def test_p3_llama2_table():
    t = G["p3_llama2"]; m = t["model"]
    fp16 = sizes.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], t["tokens"], 2)
    assert abs(fp16 / 1e9 - t["approx_fp16_GB"]) / t["approx_fp16_GB"] < 0.06
    for fmt, bits in (("int8", 8), ("int4", 4), ("int2", 2)):
        ratio = sizes.kv_cache_bytes(1, 1, 1, 1, bits / 8) / sizes.kv_cache_bytes(1, 1, 1, 1, 2)
        assert ratio == t["table_GB"][fmt] / t["table_GB"]["fp16"]


def test_p1_llama3_70b():
    t = G["p1_llama3_70b"]; m = t["model"]
    one = sizes.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], t["tokens"], t["bytes_per_value"])
    assert one == 5 * GiB
    assert 8 * one > t["over_GB"] * 1e9 and 7 * one < t["over_GB"] * 1e9


def test_stored_bytes_include_metadata():
    # 4-bit codes + one fp16 (S, Z) pair per 64 values = 4.5 bits; NVFP4: 4 + 8/16 bits
    assert sizes.stored_bytes_per_token("int4") == 2 * 128 * 4.5 / 8
    assert sizes.stored_bytes_per_token("nvfp4") == 2 * 128 * 4.5 / 8
    assert sizes.stored_bytes_per_token("int2") == 2 * 128 * 2.5 / 8
    assert sizes.stored_bytes_per_token("int8") == 2 * 128 * 8.5 / 8
    assert sizes.stored_bytes_per_token("fp16") == 512
    assert sizes.stored_bytes_per_token("fp8") == 256            # fixed scale: no metadata
    # groups of 32 / 128: one fp16 (S, Z) pair per 32 / 128 values = 5 / 4.25 bits for INT4
    assert sizes.stored_bytes_per_token("int4g32") == 2 * 128 * 5 / 8
    assert sizes.stored_bytes_per_token("int4g128") == 2 * 128 * 4.25 / 8
    assert sizes.stored_bytes_per_token("int2g32") == 2 * 128 * 3 / 8
    # per-channel K: one (S, Z) pair per dim per 128 tokens (4 bytes per 128 values) + V in groups of 64
    assert sizes.stored_bytes_per_token("int4kc") == 128 * (4 + 32 / 128) / 8 + 128 * 4.5 / 8
    # MXFP4: 4-bit codes + one byte per 32 values = 4.25 bits
    assert sizes.stored_bytes_per_token("mxfp4") == 2 * 128 * 4.25 / 8
    # the page's FP8 row: 32 layers / 8 kv heads / 32K tokens at one byte per value = 2 GiB
    assert sizes.packed_cache_bytes("fp8", 32, 8, 32768) == 2 * GiB
    # and its FP16 column (4 / 16 / 32 GiB at 32K / 128K / 256K): the fp16 block holds exactly
    # the raw values
    for T, gib in ((32768, 4), (131072, 16), (262144, 32)):
        assert sizes.packed_cache_bytes("fp16", 32, 8, T) == gib * GiB
    # 4 GiB fp16 at 32 layers / 8 kv heads / 32K tokens is 1 GiB at 4 bits before metadata
    assert sizes.packed_cache_bytes("int4", 32, 8, 32768) == 1 * GiB * 4.5 / 4
