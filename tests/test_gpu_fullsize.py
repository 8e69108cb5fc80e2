"""GPU parity at the full per-layer sizes of the five workloads, in the launch configuration the
bench times (same batch, kv heads, query heads and cached length, hence the same work split).

Inputs are drawn on the GPU with the seeded device generator; the sampled (batch, kv_head)
slices are copied to the host and the oracle recomputes from them.  Checked per workload:
  * packed bytes of sampled blocks (first, middle, last of each tier) bit-exact;
  * decode output of sampled (batch, kv_head) pairs within 1e-3 * max|out| (fp32 output).
One layer per workload: layers are independent and share the kernel configuration."""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import kvq_synth as syn
from oracle.cache import LayerCache
from oracle.attention import decode_layer
from oracle import layout as olayout
from oracle.quant import quantize_tokens, affine_params, k_per_channel

pytestmark = pytest.mark.gpu

SIGMA = 1.0 / np.sqrt(128.0)


def _pairs(B, H, n):
    cand = [(0, 0), (B - 1, H - 1), (B // 2, (H - 1) // 2), (0, H - 1), (B - 1, 0)]
    return list(dict.fromkeys(cand))[:n]


def _check_blocks(cache, ora: LayerCache, b, h, tier, region):
    """Bytes of the first, a middle and the last block of a tier of pair (b, h)."""
    _, nb, ntok = cache.layout(0, region)
    if ntok == 0:
        return 0
    dev = cache.region_tensor(0, region)
    fmt = ora.tier_format(tier)
    bb = olayout.block_bytes(fmt)
    K, V = ora.history(0, 0)                     # the oracle holds only this pair
    pos = np.asarray(ora.tier_tokens(tier), dtype=np.int64)
    nblk = -(-ntok // 128)
    for blk in sorted({0, nblk // 2, nblk - 1}):
        sl = pos[128 * blk:128 * (blk + 1)]
        kq, vq = quantize_tokens(K[sl], fmt, "k"), quantize_tokens(V[sl], fmt, "v")
        if k_per_channel(fmt):               # one whole 128-token window per block
            want = olayout.pack_affine_kc_block(affine_params(fmt)[0], {"codes": kq["codes"], "S": kq["S"][0],
                                                                       "Z": kq["Z"][0]}, vq)
        elif fmt == "nvfp4":
            want = olayout.pack_nvfp4_block(kq, vq, sl.size)
        elif fmt == "mxfp4":
            want = olayout.pack_mxfp4_block(kq, vq, sl.size)
        elif fmt == "fp8":
            want = olayout.pack_fp8_block(kq, vq, sl.size)
        elif fmt == "fp16":
            want = olayout.pack_fp16_block(kq, vq, sl.size)
        else:
            n, gs = affine_params(fmt)
            want = olayout.pack_affine_block(n, kq, vq, sl.size, gs)
        got = dev[b, h, blk * bb:(blk + 1) * bb].cpu().numpy()
        assert np.array_equal(got, want), f"{tier} block {blk} of (b={b}, h={h}) differs"
    return 1


def _run(cid, fmt=None, steps=1, n_pairs=2, check_steps=(1,)):
    W = syn.WORKLOADS[cid]
    fmt = fmt or W.fmt
    B, H, Hq, T, R = W.batch, W.num_kv_heads, W.num_q_heads, W.prefill, W.residual_len
    per_step = max(1, W.append_per_step)
    cache = kvq.Cache(kvq.make_config(1, B, H, T + steps * per_step + 1, fmt, R, W.old_fmt, W.old_after))
    pairs = _pairs(B, H, n_pairs)
    k = syn.draw_k_dev(cid, 0, B, H, T, W.kdist)
    v = syn.draw_v_dev(cid, 0, B, H, T)
    host = {bh: ([k[bh].cpu().numpy()], [v[bh].cpu().numpy()]) for bh in pairs}
    cache.append(0, k, v)
    del k, v
    ws = torch.empty(cache.workspace_bytes(Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    G = Hq // H
    checked = 0
    for s in range(steps):
        kn = syn.draw_k_dev(cid, 0, B, H, per_step, W.kdist, syn.STREAM_K_APPEND, s)
        vn = syn.draw_v_dev(cid, 0, B, H, per_step, syn.STREAM_V_APPEND, s)
        for bh in pairs:
            host[bh][0].append(kn[bh].cpu().numpy())
            host[bh][1].append(vn[bh].cpu().numpy())
        cache.append(0, kn, vn)
        if s + 1 not in check_steps:
            continue
        q = syn.draw_q_dev(cid, 0, B, Hq, s)
        cache.decode(0, q, SIGMA, out, ws)
        torch.cuda.synchronize()
        got_all = out.cpu().numpy().astype(np.float64)
        q_h = q.cpu().numpy()
        for (b, h) in pairs:
            ora = LayerCache(fmt, R, W.old_fmt, W.old_after)
            for kc, vc in zip(*host[(b, h)]):
                ora.append(kc[None, None], vc[None, None])
            want = decode_layer(ora, q_h[b:b + 1, h * G:(h + 1) * G], SIGMA)[0]
            got = got_all[b, h * G:(h + 1) * G]
            err = np.abs(got - want).max() / np.abs(want).max()
            assert np.isfinite(got).all() and err <= 1e-3, f"step {s + 1} (b={b}, h={h}): rel err {err:.2e}"
            if s + 1 == check_steps[-1]:
                checked += _check_blocks(cache, ora, b, h, "young", kvq.REGION_YOUNG)
                checked += _check_blocks(cache, ora, b, h, "old", kvq.REGION_OLD)
    assert checked > 0


def test_fullsize_single_layer_gqa4_1k_int4():
    _run(1, n_pairs=5)


def test_fullsize_llama2_mha_1k_int4_flush():
    _run(2, n_pairs=4)


def test_fullsize_llama3_70b_gqa8_32k_nvfp4():
    _run(3, n_pairs=2)


def test_fullsize_long_context_128k_int4():
    _run(4, "int4", steps=2, n_pairs=2, check_steps=(1, 2))


def test_fullsize_long_context_128k_int2():
    _run(4, "int2", steps=1, n_pairs=2)


def test_fullsize_long_context_128k_fp8():
    _run(4, "fp8", steps=1, n_pairs=2)


def test_fullsize_llama3_70b_gqa8_32k_fp8():
    _run(3, "fp8", n_pairs=2)


def test_fullsize_long_context_128k_int4_groups_of_32():
    _run(4, "int4g32", steps=1, n_pairs=2)


def test_fullsize_long_context_128k_int4_per_channel_k():
    _run(4, "int4kc", steps=2, n_pairs=2, check_steps=(1, 2))


def test_fullsize_long_context_128k_int4_groups_of_128():
    _run(4, "int4g128", steps=1, n_pairs=2)


def test_fullsize_long_context_128k_mxfp4():
    _run(4, "mxfp4", steps=1, n_pairs=2)


def test_fullsize_llama3_70b_gqa8_32k_mxfp4():
    _run(3, "mxfp4", n_pairs=2)


def test_fullsize_long_context_128k_fp16():
    _run(4, "fp16", steps=1, n_pairs=2)


def test_fullsize_llama3_70b_gqa8_32k_fp16():
    _run(3, "fp16", n_pairs=2)


def test_fullsize_256k_prefill_int2_int4_tiers():
    _run(5, steps=16, n_pairs=2, check_steps=(1, 16))
