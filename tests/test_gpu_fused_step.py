"""GPU: kvq_append_decode_attn (one decode step in one call) against kvq_append followed by
kvq_decode_attn on a twin cache: bitwise equal outputs and stored bytes (deterministic split),
and within the attention tolerance of the oracle.  Steps cross residual flushes, append
several tokens at once, and decode without appending.  An NVFP4 cache without a residual
appends a one-token step inside the decode launch (page "NVFP4 KV缓存技术详解" §2.1, the
update phase): its bytes are compared exactly, its output within the attention tolerance."""
import zlib

import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
from gpu_helpers import Pair, to_dev, assert_attention_close
from oracle.attention import decode_layer
from oracle import layout as olayout

pytestmark = pytest.mark.gpu

SIGMA = 1 / np.sqrt(128)
CASES = [("int4", 128, None, 0, False), ("nvfp4", 0, None, 0, False), ("fp8", 16, None, 0, False),
         ("int4g32", 256, None, 0, False), ("int4kc", 128, None, 0, False), ("int4", 128, "int2", 300, False),
         ("mxfp4", 32, None, 0, False), ("int4", 128, "int2", 300, True), ("int8", 0, "nvfp4", 200, True),
         ("int2", 128, None, 0, False), ("int2", 128, "int2", 300, False)]


@pytest.mark.parametrize("fmt,R,old,old_after,demote", CASES, ids=lambda x: str(x))
def test_fused_step_matches_separate_calls(fmt, R, old, old_after, demote):
    rng = np.random.default_rng(zlib.crc32(f"{fmt}/{R}/{old}/{demote}".encode()))
    B, H, G = 2, 2, 4
    fused = Pair(1, B, H, 2000, fmt, R, old, old_after, demote)
    sep = kvq.Cache(kvq.make_config(1, B, H, 2000, fmt, R, old, old_after, demote=demote))
    for c in (fused.gpu, sep):
        c.set_deterministic(True)
    k0 = rng.standard_normal((B, H, 300, 128)).astype(np.float16)
    v0 = rng.standard_normal((B, H, 300, 128)).astype(np.float16)
    fused.append(0, k0, v0)
    sep.append(0, to_dev(k0), to_dev(v0))
    ws = torch.empty(fused.gpu.workspace_bytes(H * G), dtype=torch.uint8, device="cuda")
    for n in [1, 1, 3, 0, 130, 1, 255, 1, 1]:
        k = rng.standard_normal((B, H, n, 128)).astype(np.float16)
        v = rng.standard_normal((B, H, n, 128)).astype(np.float16)
        q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
        out_f = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
        out_s = torch.empty_like(out_f)
        kd, vd, qd = to_dev(k), to_dev(v), to_dev(q)
        fused.gpu.append_decode(0, kd, vd, qd, SIGMA, out_f, ws)
        fused.ora[0].append(k, v)
        if n:
            sep.append(0, kd, vd)
        sep.decode(0, qd, SIGMA, out_s, ws)
        torch.cuda.synchronize()
        if fmt == "nvfp4" and R == 0 and n == 1:
            # the launch appends the token itself and attends to it as a one-token residual: the
            # same values summed in another order
            assert_attention_close(out_f.cpu().numpy().astype(np.float64), out_s.cpu().numpy().astype(np.float64))
        else:
            assert torch.equal(out_f, out_s), f"step of {n} tokens: fused and separate outputs differ"
        assert fused.gpu.seq_len(0) == sep.seq_len(0)
        fused.check_bytes(0)                              # both tiers and the residual against the oracle
        for region, tfmt in ((1, fmt), (2, old or fmt)):     # the twin's written blocks equal the fused cache's
            ntok = fused.gpu.layout(0, region)[2]
            assert fused.gpu.first_block(0, region) == sep.first_block(0, region)
            nb = (fused.gpu.first_block(0, region) + -(-ntok // 128)) * olayout.block_bytes(tfmt)
            a, b = fused.gpu.region_tensor(0, region), sep.region_tensor(0, region)
            assert torch.equal(a[..., :nb], b[..., :nb]), f"region {region} differs after a step of {n}"
        assert_attention_close(out_f.cpu().numpy().astype(np.float64), decode_layer(fused.ora[0], q, SIGMA))
    if demote:
        assert fused.ora[0].sched.young_head > 0, "the steps never demoted a block"


@pytest.mark.parametrize("G", [8, 4])
def test_nvfp4_in_launch_append(G):
    """NVFP4 without a residual, one token per step, the decode launch quantizing it: from an
    empty cache (the first step has nothing to stream), then across a block boundary (a token
    that opens a block clears it first) and on into the next block; bytes exact against the
    oracle and the twin that appends separately, attention within the tolerance."""
    rng = np.random.default_rng(90 + G)
    B, H = 2, 2
    fused = Pair(1, B, H, 600, "nvfp4", 0)
    sep = kvq.Cache(kvq.make_config(1, B, H, 600, "nvfp4", 0))
    ws = torch.empty(fused.gpu.workspace_bytes(H * G), dtype=torch.uint8, device="cuda")
    # stale bytes in the arena: a block opened by the launch must not keep them
    fused.gpu.region_tensor(0, 1).fill_(0x7F)
    sep.region_tensor(0, 1).fill_(0x7F)
    plan = [1, 1, 124, 1, 1, 1, 1, 1, 130, 1, 1]
    for n in plan:
        k = (rng.standard_normal((B, H, n, 128)) * np.where(rng.random(128) < 0.03, 20.0, 1.0)).astype(np.float16)
        v = rng.standard_normal((B, H, n, 128)).astype(np.float16)
        q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
        kd, vd, qd = to_dev(k), to_dev(v), to_dev(q)
        out_f = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
        out_s = torch.empty_like(out_f)
        fused.gpu.append_decode(0, kd, vd, qd, SIGMA, out_f, ws)
        fused.ora[0].append(k, v)
        sep.append(0, kd, vd)
        sep.decode(0, qd, SIGMA, out_s, ws)
        torch.cuda.synchronize()
        fused.check_bytes(0)
        ntok = fused.gpu.layout(0, 1)[2]
        nb = -(-ntok // 128) * olayout.block_bytes("nvfp4")
        a, b = fused.gpu.region_tensor(0, 1), sep.region_tensor(0, 1)
        assert torch.equal(a[..., :nb], b[..., :nb]), f"arena differs after {ntok} tokens"
        got = out_f.cpu().numpy().astype(np.float64)
        assert_attention_close(got, decode_layer(fused.ora[0], q, SIGMA))
        assert_attention_close(got, out_s.cpu().numpy().astype(np.float64))
    assert fused.gpu.layout(0, 1)[2] == sum(plan)
