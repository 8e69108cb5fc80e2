"""Shared helpers of the GPU parity tests: drive the HIP path and the oracle on the same inputs."""
import numpy as np
import torch

import bit_quantized_kv_kvq_amd as kvq
from oracle.cache import LayerCache
from oracle.attention import decode_layer
from oracle import layout as olayout


def adversarial_tokens(rng, B, H, n, scale=1.0):
    """fp16 [B, H, n, 128] mixing the value patterns that stress the quantizers."""
    x = rng.standard_normal((B, H, n, 128)) * scale
    kind = rng.integers(0, 9, size=(B, H, n, 2))            # per (token, 64-group)
    for g in range(2):
        sl = (Ellipsis, slice(64 * g, 64 * g + 64))
        grp = x[sl]
        k = kind[..., g][..., None]
        grp = np.where(k == 1, grp * 15.0, grp)                                    # outliers
        grp = np.where(k == 2, np.round(grp * 4) / 2, grp)                         # many exact ties
        grp = np.where(k == 3, grp[..., :1] * 0 + 1.5, grp)                        # constant group
        grp = np.where(k == 4, np.where(grp > 0, 2.5, -1.25), grp)                 # two values
        grp = np.where(k == 5, grp * 3e-6, grp)                                    # subnormal range
        grp = np.where(k == 6, np.clip(grp * 20000, -65504, 65504), grp)           # near fp16 max
        grp = np.where(k == 7, 100.0 + np.abs(grp) * 0.01, grp)                    # narrow, one-sided
        x[sl] = grp
    return x.astype(np.float16)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Pair:
    """A GPU cache and its oracle twin for one layer-set."""

    def __init__(self, layers, B, H, max_tokens, fmt, R, old_fmt=None, old_after=0, demote=False):
        self.cfg = kvq.make_config(layers, B, H, max_tokens, fmt, R, old_fmt, old_after, demote=demote)
        self.gpu = kvq.Cache(self.cfg)
        self.ora = [LayerCache(fmt, R, old_fmt, old_after, demote) for _ in range(layers)]
        self.B, self.H, self.fmt, self.old_fmt, self.R = B, H, fmt, old_fmt or fmt, R

    def append(self, layer, k16, v16):
        self.gpu.append(layer, to_dev(k16), to_dev(v16))
        self.ora[layer].append(k16, v16)

    def flush(self, layer):
        self.gpu.flush(layer)
        self.ora[layer].flush()

    def check_bytes(self, layer, bh=None):
        torch.cuda.synchronize()
        pairs = bh if bh is not None else [(b, h) for b in range(self.B) for h in range(self.H)]
        o = self.ora[layer]
        for region, tier in ((1, "young"), (2, "old")):
            _, nb, ntok = self.gpu.layout(layer, region)
            assert ntok == len(o.tier_tokens(tier))
            if ntok == 0:
                continue
            dev = self.gpu.region_tensor(layer, region)
            fmt = o.tier_format(tier)
            nblk = -(-ntok // 128)
            bb = olayout.block_bytes(fmt)
            fb = self.gpu.first_block(layer, region)        # young blocks before it were demoted
            assert fb * 128 == (o.sched.young_head if tier == "young" else 0)
            for b, h in pairs:
                got = dev[b, h, fb * bb:(fb + nblk) * bb].cpu().numpy()
                want = o.arena(b, h, tier).ravel()
                if not np.array_equal(got, want):
                    bad = np.flatnonzero(got != want)
                    raise AssertionError(f"{tier} arena (b={b}, h={h}, fmt={fmt}): {bad.size} bytes differ, "
                                         f"first at {bad[:8]} got {got[bad[:8]]} want {want[bad[:8]]}")
        if self.R:
            dev = self.gpu.region_tensor(layer, 0)
            for b, h in pairs:
                data, mask = o.residual(b, h)
                got = dev[b, h].cpu().numpy()
                assert np.array_equal(got[mask], data[mask]), f"residual (b={b}, h={h})"

    def decode(self, layer, q16, sigma, b_list=None, out_dtype=torch.float32):
        Hq = q16.shape[1]
        ws = torch.empty(self.gpu.workspace_bytes(Hq), dtype=torch.uint8, device="cuda")
        out = torch.empty((self.B, Hq, 128), dtype=out_dtype, device="cuda")
        self.gpu.decode(layer, to_dev(q16), sigma, out, ws)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        want = decode_layer(self.ora[layer], q16, sigma, b_list)
        return got, want


def assert_attention_close(got, want, tol=1e-3, b_list=None):
    if b_list is not None:
        got, want = got[b_list], want[b_list]
    err = np.abs(got - want).max()
    ref = np.abs(want).max()
    assert np.isfinite(got).all(), "non-finite output"
    assert err <= tol * ref, f"max|d| {err:.3e} > {tol} * max|out| {ref:.3e} (ratio {err / ref:.2e})"
    return err / ref
