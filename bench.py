"""Decode-step benchmark of the quantized KV cache on one MI355X.

A step is, for every layer: append the step's new token(s) (quantize + pack when the fp16
residual is full or the residual length is 0, else an fp16 copy into the residual) and one
fused dequant + decode-attention call over the whole cache.  Inputs are seeded synthetic K/V/Q
drawn on the GPU before the timed region.

Headline workload: 32 layers, batch 8, 32 query / 8 KV heads, head_dim 128, 131072 cached
tokens per sequence in INT4 affine (group 64, fp16 S/Z, 128-token fp16 residual), Student-t
(nu = 4) K and Gaussian V, consecutive decode steps with append and residual flushes.  The
prefill is sized so that the first timed step is the one that flushes the full residual.

Output: one JSON line.  `value` is the effective HBM GB/s of the cache read (codes + scales +
zero points + fp16 residual) summed over the timed steps, divided by their wall time.
`roofline` gives the decode-attention call alone, timed with HIP events on the stream it is
launched on.  `cpu_baseline` times the CPU oracle on a bounded sample of the same workload, on
a pool of host processes.  With no --workload, `per_config` holds the other workloads measured
in the same run: the 1K single layer (MALL-hot and cold), the Llama-2-shaped MHA step, the
32K NVFP4 GQA-8 step, the 128K INT2 step and the 256K tier workload with its bulk prefill.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DECODE_SRC = os.path.join(ROOT, "bit_quantized_kv_kvq_amd", "csrc", "kvq_decode.hip")
POOL_CAP = 16           # host worker processes at most (one GPU's share of a box's cores)

# workload name -> (config id in kvq_synth.WORKLOADS, young format override)
WORKLOADS = {
    "c1": (1, None), "c2": (2, None), "c3": (3, None),
    "c4-int4": (4, "int4"), "c4-int2": (4, "int2"), "c5": (5, None),
    "c4-int4g32": (4, "int4g32"), "c4-int4g128": (4, "int4g128"), "c4-int4kc": (4, "int4kc"),
    "c3-mxfp4": (3, "mxfp4"), "c4-mxfp4": (4, "mxfp4"), "c3-fp8": (3, "fp8"), "c4-fp8": (4, "fp8"), "c3-fp16": (3, "fp16"), "c4-fp16": (4, "fp16"),
    "c5-demote": (5, None), "c4-ragged": (4, "int4"),
}
# ragged workloads: sequence b of the batch holds T (b + 1) / batch of the workload's T tokens
RAGGED = {"c4-ragged"}
# workloads whose young blocks move to the old tier as they age (demote_young), and the
# timed steps they default to (a block of one (batch, kv_head) ages every 128 one-token steps)
DEMOTE_STEPS = {"c5-demote": 320}
# the other workloads of a default run: (steps, warmup, (batch, kv_head) pairs for the oracle)
PER_CONFIG = [("c2", 8, 2, 32), ("c3", 8, 2, 12), ("c4-int2", 20, 5, 32), ("c5", 16, 0, 8)]


def bytes_per_token(fmt: str) -> float:
    """Stored bytes of one token of one (batch, kv_head), K and V together."""
    m = re.fullmatch(r"int([248])(?:g(32|64|128)|(kc))?", fmt)
    if m:   # n-bit codes + one fp16 (S, Z) pair per group of K and of V
        n, gs = int(m.group(1)), int(m.group(2) or 64)
        if m.group(3):   # K per channel: one pair per dim per 128-token block
            return (4096 * n + 1536) / 128
        return (4096 * n + 1024 * (128 // gs)) / 128
    return {"nvfp4": 18432 / 128, "mxfp4": 17408 / 128, "fp8": 32768 / 128, "fp16": 512.0}[fmt]


def decode_bytes(cache, layer: int, fmt: str, old_fmt: str, ragged: bool = False) -> float:
    """Algorithmic cache bytes one decode call reads: every cached token once."""
    import bit_quantized_kv_kvq_amd as kvq
    B, H = cache.cfg.batch, cache.cfg.num_kv_heads
    if ragged:
        tot = 0.0
        for b in range(B):
            i = cache.seq_info(layer, b)
            tot += H * (i["old_tokens"] * bytes_per_token(old_fmt) + i["young_tokens"] * bytes_per_token(fmt)
                        + i["residual"] * 512.0)
        return tot
    n_res = cache.layout(layer, kvq.REGION_RESIDUAL)[2]
    n_young = cache.layout(layer, kvq.REGION_YOUNG)[2]
    n_old = cache.layout(layer, kvq.REGION_OLD)[2]
    return B * H * (n_old * bytes_per_token(old_fmt) + n_young * bytes_per_token(fmt) + n_res * 512.0)


def kernel_src_sha() -> str:
    return hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per decode launch from the committed PMC summary, when it was taken on the
    current decode kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"kernel_src_sha:\s*([0-9a-f]+)", txt)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not sha or not val or sha.group(1) != kernel_src_sha():
        return None
    return float(val.group(1))


# ----------------------------------------------------------------------------- CPU oracle pool

def _worker_ready(_):
    return os.getpid()


def oracle_task(spec):
    """One (batch, kv_head) pair of layer 0 through the CPU oracle: quantize every token it
    received (chunks in order, as the GPU cache did) and attend in float64.  Runs in a worker
    process (one BLAS thread).  Returns (seconds, out [G, 128] float64, algorithmic bytes)."""
    from threadpoolctl import threadpool_limits
    from oracle.cache import LayerCache
    from oracle.attention import decode_layer
    fmt, R, old_fmt, old_after, demote, kch, vch, q16, sigma = spec
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        lc = LayerCache(fmt, R, old_fmt, old_after, demote)
        for kc, vc in zip(kch, vch):
            lc.append(kc[None, None], vc[None, None])
        out = decode_layer(lc, q16[None], sigma)[0]
        dt = time.perf_counter() - t0
    nb = (len(lc.sched.old) * bytes_per_token(lc.old_fmt) + len(lc.tier_tokens("young")) * bytes_per_token(lc.fmt)
          + len(lc.sched.residual) * 512.0)
    return dt, out, nb


def start_pool():
    """Worker processes for the oracle, all forked here, before this process touches the GPU
    (torch is not imported yet), so that no worker holds GPU state; they live until the pool
    is closed.  At most POOL_CAP workers, and no more than the cores this process may run on."""
    import multiprocessing as mp
    n = max(1, min(POOL_CAP, len(os.sched_getaffinity(0))))
    pool = mp.get_context("fork").Pool(n)
    pids = set(pool.map(_worker_ready, range(4 * n), chunksize=1))
    return pool, n, len(pids)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_oracle(pool, specs, gpu_outs):
    """Oracle on the sampled pairs in the pool: (wall seconds, summed worker seconds, bytes,
    max |gpu - oracle| / max |oracle| over the samples)."""
    t0 = time.perf_counter()
    res = pool.map(oracle_task, specs, chunksize=1)
    wall = time.perf_counter() - t0
    worst = 0.0
    for (dt, want, nb), got in zip(res, gpu_outs):
        worst = max(worst, float(np.abs(got - want).max() / np.abs(want).max()))
    return wall, sum(r[0] for r in res), sum(r[2] for r in res), worst


# ----------------------------------------------------------------------------- probes

def copy_probe():
    """A plain copy of a known size (1 GiB), for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n, "launches": 5}))


def read_probe_gbs() -> float:
    """Achievable HBM read rate of one launch: the library's read probe (a grid-stride stream of
    16-byte loads) over a 4 GiB buffer, timed with HIP events on its stream, best of 6."""
    import torch
    import bit_quantized_kv_kvq_amd as kvq
    x = torch.zeros(1 << 32, dtype=torch.uint8, device="cuda")
    sink = torch.empty(kvq.read_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.read_probe(x, sink)
        e1.record()
        e1.synchronize()
        best = max(best, x.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, sink
    torch.cuda.empty_cache()
    return best


def same_bytes_probe_us(nbytes: float) -> float:
    """Event-timed duration of the library's read probe over a buffer of the decode call's
    algorithmic bytes (median of 24 launches, rotated over copies that together exceed the
    256 MiB MALL): what one streaming launch of that size reaches on this machine, launch cost
    included, as the decode launches are timed."""
    import torch
    import bit_quantized_kv_kvq_amd as kvq
    n = max(16, int(nbytes) // 16 * 16)
    bufs = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(max(1, -(-600 << 20) // n))]
    sink = torch.empty(kvq.read_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
    for b in bufs:
        kvq.read_probe(b, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(24)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        kvq.read_probe(bufs[i % len(bufs)], sink)
        e1.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    del bufs, sink
    torch.cuda.empty_cache()
    return ts[len(ts) // 2]


NOISE_FORMATS = ("int8", "fp8", "int4g32", "int4", "int4kc", "int4g128", "nvfp4", "mxfp4", "int2g32", "int2kc", "int2")


def noise_study(lengths, n_queries: int):
    """Quantization noise of each cache format against sequence length (the comparison of
    page "NVFP4 KV缓存技术详解" §3.2, NVFP4 against MXFP4 over long sequences, on synthetic data).

    For the K distributions of the 128K workload (Student-t, nu = 4) and of the 32K NVFP4 workload
    (Gaussian, 3 outlier channels x20), V Gaussian: one sequence of 8 kv heads grows through the
    given lengths; at each length every format's cache (residual 0: every token quantized)
    answers the same n_queries decode calls of 32 query heads (GQA 4), and the error is
    ||o_fmt - o_fp16|| / ||o_fp16|| over heads and queries, o_fp16 being the same kernel on the
    fp16 cache (itself within the parity tolerance of exact attention).  One JSON line per K
    distribution."""
    import torch
    import bit_quantized_kv_kvq_amd as kvq
    import kvq_synth as syn
    sigma = 1.0 / np.sqrt(128.0)
    H, G = 8, 4
    Lmax = max(lengths)
    for cid in (4, 3):
        W = syn.WORKLOADS[cid]
        k = syn.draw_k_dev(cid, 0, 1, H, Lmax, W.kdist)
        v = syn.draw_v_dev(cid, 0, 1, H, Lmax)
        qs = [syn.draw_q_dev(cid, 0, 1, H * G, s) for s in range(n_queries)]
        outs = {}
        for fmt in ("fp16",) + NOISE_FORMATS:
            # per-channel K fills 128-token windows through the residual; a flush after each
            # append (the lengths are whole windows) leaves every token quantized, as R = 0 does
            R = 128 if fmt.endswith("kc") else 0
            cache = kvq.Cache(kvq.make_config(1, 1, H, Lmax, fmt, R))
            ws = torch.empty(cache.workspace_bytes(H * G), dtype=torch.uint8, device="cuda")
            done = 0
            for L in sorted(lengths):
                cache.append(0, k[:, :, done:L].contiguous(), v[:, :, done:L].contiguous())
                if R:
                    cache.flush(0)
                done = L
                o = torch.empty((n_queries, H * G, 128), dtype=torch.float32, device="cuda")
                for i, q in enumerate(qs):
                    cache.decode(0, q, sigma, o[i:i + 1], ws)
                outs[(fmt, L)] = o.double()
            torch.cuda.synchronize()
            del cache, ws
        errs = {fmt: {str(L): float((outs[(fmt, L)] - outs[("fp16", L)]).norm() / outs[("fp16", L)].norm())
                      for L in lengths} for fmt in NOISE_FORMATS}
        kd = W.kdist
        desc = (f"student-t nu={kd.nu:g}" if kd.kind == "student_t" else "normal") + \
            (f", {kd.outlier_channels} outlier channels x{kd.outlier_scale:g}" if kd.outlier_channels else "")
        print(json.dumps({"study": "decode output error vs fp16 cache", "k_distribution": desc,
                          "lengths": list(lengths), "queries": n_queries, "kv_heads": H, "gqa": G,
                          "relative_error": errs}), flush=True)
        del k, v, qs, outs
        torch.cuda.empty_cache()


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- one workload

def measure(name: str, steps: int, warmup: int, n_pairs: int, separate_append: bool = False):
    """Prefill, warm up, time `steps` decode steps of workload `name`.

    Returns (result dict, oracle specs of the sampled pairs, GPU fp32 outputs of those pairs).
    With a residual and one token per step, the prefill holds T - warmup - k tokens (k = half the
    timed steps), so that the residual is full when the cache holds the workload's T tokens, at
    timed step k: that step flushes it in every layer (reported as flush_step_ms; the step is in
    the middle of the timed run, where the GPU's clocks have settled)."""
    import torch
    import bit_quantized_kv_kvq_amd as kvq
    import kvq_synth as syn

    demote = name in DEMOTE_STEPS
    ragged = name in RAGGED
    cid, fmt_over = WORKLOADS[name]
    W = syn.WORKLOADS[cid]
    fmt = fmt_over or W.fmt
    old_fmt = W.old_fmt or fmt
    L, B, Hq, H, T, R = W.num_layers, W.batch, W.num_q_heads, W.num_kv_heads, W.prefill, W.residual_len
    G = Hq // H
    sigma = 1.0 / np.sqrt(128.0)
    per_step = max(1, W.append_per_step)
    n_steps = warmup + steps
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    flush_k = min(steps // 2, R - 1 - warmup) if R > 0 else -1
    flush_first = R > 0 and per_step == 1 and not ragged and not demote and flush_k >= 0
    # NVFP4 without a residual: kvq_append_decode_attn quantizes a one-token step inside the
    # decode launch (one call and one launch per layer)
    in_launch = fmt == "nvfp4" and R == 0 and not W.old_after and not demote and per_step == 1
    T0 = T - warmup - flush_k if flush_first else T

    # the process loads each kernel's code on its first launch, a one-time cost that belongs
    # to neither the prefill rate nor a step: a 300-token append and a decode on a scratch
    # cache of one kv head load them first
    scratch = kvq.Cache(kvq.make_config(1, 1, 1, 512, fmt, R))
    scratch.append(0, torch.zeros((1, 1, 300, 128), dtype=torch.float16, device=dev),
                   torch.zeros((1, 1, 300, 128), dtype=torch.float16, device=dev))
    sws = torch.empty(scratch.workspace_bytes(G), dtype=torch.uint8, device=dev)
    sq = torch.zeros((1, G, 128), dtype=torch.float16, device=dev)
    sout = torch.empty((1, G, 128), dtype=torch.float16, device=dev)
    scratch.decode(0, sq, sigma, sout, sws)
    torch.cuda.synchronize()

    cfg = kvq.make_config(L, B, H, T0 + n_steps * per_step + 9, fmt, R, W.old_fmt, W.old_after, demote=demote)
    cache = kvq.Cache(cfg)
    samples_bh = [(b, h) for b in range(B) for h in range(H)][:n_pairs]
    host_hist = {bh: ([], []) for bh in samples_bh}
    lens = [T0 * (b + 1) // B for b in range(B)] if ragged else [T0] * B
    if ragged:
        assert W.old_after == 0 and R > 0, "the ragged step tracker models one tier with a residual"

    # ---- untimed state: bulk prefill of every layer (one append of T0 tokens, or one per
    # sequence when ragged); HIP events around each layer's appends give the bulk quantize rate
    # (fp16 read + packed bytes written)
    t_prefill = time.perf_counter()
    pre_events = []
    for l in range(L):
        k = syn.draw_k_dev(cid, l, B, H, T0, W.kdist)
        v = syn.draw_v_dev(cid, l, B, H, T0)
        if l == 0:
            for (b, h) in samples_bh:
                host_hist[(b, h)][0].append(k[b, h, :lens[b]].cpu().numpy())
                host_hist[(b, h)][1].append(v[b, h, :lens[b]].cpu().numpy())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if ragged:
            for b in range(B):
                cache.append_seq(l, b, k[b, :, :lens[b]].contiguous(), v[b, :, :lens[b]].contiguous())
        else:
            cache.append(l, k, v)
        e1.record(stream)
        pre_events.append((e0, e1))
        del k, v
        if l % 16 == 15 or l == L - 1:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t_prefill
    # one more decode on the scratch cache: in a kernel trace the launches between the two
    # scratch decodes are the prefill's, those after the second one the steps'
    scratch.decode(0, sq, sigma, sout, sws)
    torch.cuda.synchronize()
    del scratch, sws, sq, sout
    pre_ms = float(sum(a.elapsed_time(b) for a, b in pre_events))
    pre_bytes = float(L * H * sum(lens) * 2 * 128 * 2) + sum(decode_bytes(cache, l, fmt, old_fmt, ragged)
                                                                for l in range(L))
    if ragged:
        track = [[[cache.seq_info(l, b)["young_tokens"], cache.seq_info(l, b)["residual"]] for b in range(B)]
                 for l in range(L)]
        bpt = bytes_per_token(fmt)

    # ---- step inputs, resident in HBM before the timed region
    knew = [[syn.draw_k_dev(cid, l, B, H, per_step, W.kdist, syn.STREAM_K_APPEND, s) for l in range(L)]
            for s in range(n_steps)]
    vnew = [[syn.draw_v_dev(cid, l, B, H, per_step, syn.STREAM_V_APPEND, s) for l in range(L)]
            for s in range(n_steps)]
    qs = [[syn.draw_q_dev(cid, l, B, Hq, s) for l in range(L)] for s in range(n_steps)]
    for s in range(n_steps):
        for (b, h) in samples_bh:
            host_hist[(b, h)][0].append(knew[s][0][b, h].cpu().numpy())
            host_hist[(b, h)][1].append(vnew[s][0][b, h].cpu().numpy())
    ws = torch.empty(cache.workspace_bytes(Hq), dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, Hq, 128), dtype=torch.float16, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    # HIP events, all created (and each recorded once) before the timed region: around each
    # timed step; around one decode launch per timed step (layer s mod L of step s) and around
    # the separate append of that layer when the step makes one.  Events around every launch
    # would cost about 3 % of the step time themselves (measured).
    def mk(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    step_ev, dec_ev, app_ev = mk(steps), mk(steps), mk(steps)
    dem_ev = mk(L * (steps * per_step // 128 + 2) if demote else 0)
    for e0, e1 in step_ev + dec_ev + app_ev + dem_ev:
        e0.record(stream)
        e1.record(stream)
    app_used, dem_used = [], []

    def demotes(l):
        if not demote:
            return False
        n_old = cache.layout(l, kvq.REGION_OLD)[2]
        return (cache.layout(l, kvq.REGION_YOUNG)[2] >= 128
                and n_old + 128 <= cache.seq_len(l)[0] + per_step - W.old_after)

    timed_bytes = []

    def step(s, i=None, nbytes=None):
        timed = s % L if i is not None else -1
        if i is not None:
            step_ev[i][0].record(stream)
        for l in range(L):
            if ragged:
                quantizes = any(t[1] + per_step > R for t in track[l])
                for t in track[l]:
                    if t[1] + per_step > R:
                        t[0] += t[1] + per_step - ((t[1] + per_step - 1) % R + 1)
                        t[1] = (t[1] + per_step - 1) % R + 1
                    else:
                        t[1] += per_step
            else:
                quantizes = (R == 0 and not in_launch) or (R > 0 and cache.seq_len(l)[1] + per_step > R) or demotes(l)
            # one kvq_append_decode_attn call per layer: its decode launch copies the tokens
            # that go to the residual itself, after the quantize launch of a step that flushes.
            # The layer whose launches are event-timed in a flushing step (and a demoting one)
            # makes the two calls separately, so that the append and the decode are timed apart.
            if separate_append or (quantizes and (l == timed or demotes(l))):
                dem = nbytes is not None and demotes(l) and len(dem_used) < len(dem_ev)
                if dem:
                    fb = cache.first_block(l, kvq.REGION_YOUNG)
                    dem_ev[len(dem_used)][0].record(stream)
                if l == timed:
                    app_ev[i][0].record(stream)
                cache.append(l, knew[s][l], vnew[s][l])
                if l == timed:
                    app_ev[i][1].record(stream)
                    app_used.append(i)
                if dem:
                    dem_ev[len(dem_used)][1].record(stream)
                    dem_used.append(cache.first_block(l, kvq.REGION_YOUNG) - fb)
                if l == timed:
                    dec_ev[i][0].record(stream)
                cache.decode(l, qs[s][l], sigma, outs[l], ws)
            else:
                if l == timed:
                    dec_ev[i][0].record(stream)
                cache.append_decode(l, knew[s][l], vnew[s][l], qs[s][l], sigma, outs[l], ws)
            if l == timed:
                dec_ev[i][1].record(stream)
            if nbytes is not None:
                nbytes.append(H * sum(t[0] * bpt + t[1] * 512.0 for t in track[l]) if ragged
                              else decode_bytes(cache, l, fmt, old_fmt))
                if l == timed:
                    timed_bytes.append(nbytes[-1])
        if i is not None:
            step_ev[i][1].record(stream)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    if flush_first:
        assert cache.seq_len(0) == (T - flush_k, R - flush_k), cache.seq_len(0)

    nbytes = []
    gc.collect()
    gc.disable()            # no collector pause inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, s in enumerate(range(warmup, n_steps)):
        step(s, i, nbytes)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    if ragged:
        for l in range(L):
            assert sum(H * (t[0] * bpt + t[1] * 512.0) for t in track[l]) == decode_bytes(cache, l, fmt, old_fmt, True)

    # the 1-token append as a call of its own, on the last layer after the timed steps (R = 0:
    # the quantize launch that an in-launch append saves)
    sep_app = []
    if in_launch:
        for s in range(min(8, n_steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            cache.append(L - 1, knew[s][L - 1], vnew[s][L - 1])
            e1.record(stream)
            sep_app.append((e0, e1))
        torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
    probe_us = same_bytes_probe_us(float(np.mean(timed_bytes)))
    dec_ms = np.array([a.elapsed_time(b) for a, b in dec_ev])
    app_ms = np.array([app_ev[i][0].elapsed_time(app_ev[i][1]) for i in app_used])
    total_bytes = float(np.sum(nbytes))
    achieved = float(np.mean(timed_bytes) / (dec_ms.mean() * 1e-3) / 1e9)
    res = {
        "workload": (W.name if fmt_over is None else W.name.replace(W.fmt, fmt))
                    + (", young blocks demoted as they age" if demote else "")
                    + (f", ragged: sequence b holds {T0}(b+1)/{B} tokens" if ragged else ""),
        "layers": L, "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": 128,
        "cached_tokens": lens if ragged else T, "format": fmt, "old_format": W.old_fmt, "residual": R,
        "append_per_step": per_step, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "steps_per_s": round(steps / wall, 2),
        "gbs": round(total_bytes / wall / 1e9, 1),
        "pct_hbm_peak": round(100 * total_bytes / wall / 1e9 / HBM_PEAK_GBS, 2),
        "decode_launch_us": round(float(dec_ms.mean()) * 1e3, 2),
        "decode_bytes_per_launch": round(float(np.mean(timed_bytes))),
        "decode_gbs": round(achieved, 1),
        "decode_frac": round(achieved / HBM_PEAK_GBS, 4),
        "read_probe_same_bytes_us": round(probe_us, 2),
        "decode_vs_read_probe": round(probe_us / (float(dec_ms.mean()) * 1e3), 3),
        "prefill_s": round(t_prefill, 2),
        "prefill_quantize_ms": round(pre_ms, 2),
        "prefill_quantize_gbs": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
        "step_event_ms_mean": round(float(step_ms.mean()), 4),
    }
    if in_launch:
        res["append_in_launch"] = True
        res["append_1_separate_us"] = round(float(np.mean([a.elapsed_time(b) for a, b in sep_app])) * 1e3, 2)
        res["append_note"] = ("each step's token is quantized inside the decode launch (kvq_append_decode_attn); "
                              "append_1_separate_us: HIP events around kvq_append of one token as a call of its own "
                              "(8 calls on the last layer after the timed steps)")
    if app_used:
        res["append_us"] = round(float(app_ms.mean()) * 1e3, 2)
        res["append_note"] = ("HIP events around one layer's kvq_append per timed step (" +
                              ("quantize of the step's token" if R == 0 else
                               "flush of the full residual + copy of the new tokens" if per_step > 1 or flush_first
                               else "residual copy") + ")")
    if app_used and R > 0 and per_step >= R:
        # every step's append flushes the full residual: its quantize rate, as the prefill's
        qbytes = B * H * R * (512 + bytes_per_token(fmt))
        res["append_quantize_gbs"] = round(qbytes / (float(app_ms.mean()) * 1e-3) / 1e9, 1)
        res["append_quantize_note"] = ("fp16 read + packed bytes written of the flushed residual over append_us "
                                       "(the same launch also copies the step's tokens into the residual)")
    if flush_first:
        res["flush_step_ms"] = round(float(step_ms[flush_k]), 4)
        res["plain_step_ms_mean"] = round(float(np.delete(step_ms, flush_k).mean()), 4) if steps > 1 else None
        res["flush_note"] = (f"timed step {flush_k} appends to a full residual in every layer: each layer's "
                             "append quantizes the 128 residual tokens into the young tier, then decodes")
        res["flush_append_us"] = (round(float(app_ms[app_used.index(flush_k)]) * 1e3, 2)
                                  if flush_k in app_used else None)
    if demote:
        blk_bytes = B * H * 128 * (bytes_per_token(fmt) + bytes_per_token(old_fmt))
        dm = np.array([dem_ev[i][0].elapsed_time(dem_ev[i][1]) for i in range(len(dem_used))])
        nblk = int(sum(dem_used))
        res["demote_young"] = 1
        res["demotion"] = {"appends": len(dem_used), "blocks": nblk,
                           "append_us": round(float(dm.mean()) * 1e3, 2) if dem_used else None,
                           "bytes_per_block": round(blk_bytes),
                           "gbs": round(blk_bytes * nblk / (dm.sum() * 1e-3) / 1e9, 1) if nblk else None,
                           "note": "event brackets around the whole append call that demotes (its residual "
                                   "copy included)"}

    # ---- parity on sampled outputs at full size: one more fp32 decode of layer 0
    out32 = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    cache.decode(0, qs[n_steps - 1][0], sigma, out32, ws)
    torch.cuda.synchronize()
    out_h = out32.cpu().numpy().astype(np.float64)
    q_h = qs[n_steps - 1][0].cpu().numpy()
    specs, gpu_outs = [], []
    for (b, h) in samples_bh:
        specs.append((fmt, R, W.old_fmt, W.old_after, demote, host_hist[(b, h)][0], host_hist[(b, h)][1],
                      q_h[b, h * G:(h + 1) * G], sigma))
        gpu_outs.append(out_h[b, h * G:(h + 1) * G])
    res["_pairs_per_step"] = L * B * H
    del cache, ws, outs, knew, vnew, qs, out32
    gc.collect()
    torch.cuda.empty_cache()
    return res, specs, gpu_outs


def measure_c1(n_copies: int = 200, reps: int = 200):
    """The 1K single-layer workload: decode of the prefilled state (1024 INT4 + 128 fp16 tokens;
    the step's token is the last residual token), MALL-hot (one cache, repeated) and cold (the
    same call rotated over n_copies caches, ~1.7 MB each, more than the 256 MiB of MALL), each
    the mean over `reps` calls between two synchronizations; then the 1-token append timed
    separately on a full residual (a flush) and on a part-filled one (an fp16 copy)."""
    import torch
    import bit_quantized_kv_kvq_amd as kvq
    import kvq_synth as syn
    cid = 1
    W = syn.WORKLOADS[cid]
    B, Hq, H, T, R = W.batch, W.num_q_heads, W.num_kv_heads, W.prefill, W.residual_len
    G = Hq // H
    sigma = 1.0 / np.sqrt(128.0)
    k = syn.draw_k_dev(cid, 0, B, H, T, W.kdist)
    v = syn.draw_v_dev(cid, 0, B, H, T)
    q = syn.draw_q_dev(cid, 0, B, Hq)
    caches = [kvq.Cache(kvq.make_config(1, B, H, T + 64, W.fmt, R)) for _ in range(n_copies)]
    for c in caches:
        c.append(0, k, v)
    ws = torch.empty(caches[0].workspace_bytes(Hq), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    nb = decode_bytes(caches[0], 0, W.fmt, W.fmt)
    for _ in range(5):
        caches[0].decode(0, q, sigma, out, ws)
    torch.cuda.synchronize()

    def timed(seq):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for c in seq:
            c.decode(0, q, sigma, out, ws)
        e1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / len(seq), e0.elapsed_time(e1) * 1e-3 / len(seq)

    hot_wall, hot_ev = timed([caches[0]] * reps)
    timed([caches[i % n_copies] for i in range(n_copies)])          # every copy read once first
    cold_wall, cold_ev = timed([caches[i % n_copies] for i in range(reps)])
    # the parity sample (fp32 out of the first cache) and the 1-token appends
    out32 = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    caches[0].decode(0, q, sigma, out32, ws)
    torch.cuda.synchronize()
    gpu = out32.cpu().numpy().astype(np.float64)
    kh, vh, qh = k.cpu().numpy(), v.cpu().numpy(), q.cpu().numpy()
    specs = [(W.fmt, R, None, 0, False, [kh[0, h]], [vh[0, h]], qh[0, h * G:(h + 1) * G], sigma) for h in range(H)]
    gpu_outs = [gpu[0, h * G:(h + 1) * G] for h in range(H)]
    app = []
    for s in range(9):
        kn = syn.draw_k_dev(cid, 0, B, H, 1, W.kdist, syn.STREAM_K_APPEND, s)
        vn = syn.draw_v_dev(cid, 0, B, H, 1, syn.STREAM_V_APPEND, s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        caches[1].append(0, kn, vn)
        e1.record()
        torch.cuda.synchronize()
        app.append(e0.elapsed_time(e1) * 1e3)
    res = {
        "workload": W.name, "layers": 1, "batch": B, "q_heads": Hq, "kv_heads": H, "cached_tokens": T,
        "format": W.fmt, "residual": R, "decode_bytes_per_launch": round(nb),
        "hot": {"decode_us": round(hot_ev * 1e6, 2), "wall_us_per_call": round(hot_wall * 1e6, 2),
                "gbs": round(nb / hot_ev / 1e9, 1), "decode_frac": round(nb / hot_ev / 1e9 / HBM_PEAK_GBS, 5),
                "steps_per_s": round(1.0 / hot_wall, 1),
                "note": f"one cache decoded {reps} times back to back (its {nb / 1e6:.2f} MB stay in the MALL)"},
        "cold": {"decode_us": round(cold_ev * 1e6, 2), "wall_us_per_call": round(cold_wall * 1e6, 2),
                 "gbs": round(nb / cold_ev / 1e9, 1), "decode_frac": round(nb / cold_ev / 1e9 / HBM_PEAK_GBS, 5),
                 "steps_per_s": round(1.0 / cold_wall, 1),
                 "note": f"calls rotated over {n_copies} copies ({n_copies * nb / 1e6:.0f} MB, above the 256 MiB MALL)"},
        "append_1_flush_us": round(app[0], 2),
        "append_1_us": round(float(np.mean(app[1:])), 2),
        "append_note": "HIP events around kvq_append of one token: first on the full residual (quantize of "
                       "the 128 residual tokens + copy), then 8 more (fp16 copy into the residual)",
        "_pairs_per_step": B * H,
    }
    del caches, ws, out, out32
    gc.collect()
    torch.cuda.empty_cache()
    return res, specs, gpu_outs


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 64; 320 for c5-demote)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="one workload alone (default: the 128K INT4 headline plus every other workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=48, help="(batch, kv_head) pairs of layer 0 for the oracle")
    ap.add_argument("--probe", choices=["copy"], default=None)
    ap.add_argument("--separate-append", action="store_true",
                    help="kvq_append then kvq_decode_attn per layer (default: kvq_append_decode_attn)")
    ap.add_argument("--study", choices=["noise"], default=None,
                    help="noise: decode error of every format against the fp16 cache vs cached length")
    ap.add_argument("--study-lengths", default="1024,4096,16384,65536,131072")
    ap.add_argument("--study-queries", type=int, default=8)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; (batch, kv_head) pairs, layers and token splits shard "
              "without exchange except a final LSE merge, which is not built here. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    want_cpu = not args.no_cpu_baseline and args.probe is None and args.study is None
    pool = None
    if want_cpu:
        pool, n_workers, n_pids = start_pool()      # before anything touches the GPU
        log(f"oracle pool: {n_workers} worker processes ({n_pids} answered)")

    import torch
    if args.probe == "copy":
        copy_probe()
        return
    if args.study == "noise":
        noise_study([int(x) for x in args.study_lengths.split(",")], args.study_queries)
        return

    name = args.workload or "c4-int4"
    per_config = args.workload is None
    if args.steps is None:
        args.steps = DEMOTE_STEPS.get(name, 64)
    torch.cuda.set_device(0)
    probe = read_probe_gbs()

    log(f"{name}: prefill, {args.warmup} warmup + {args.steps} timed steps")
    head, specs, gouts = measure(name, args.steps, args.warmup, args.cpu_pairs, args.separate_append)
    head_oracle = run_oracle(pool, specs, gouts) if want_cpu else None

    line = {
        "metric": "fused dequant+decode-attn effective GB/s (% HBM peak); decode steps/s",
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{head['format']}-codes/fp16-operands/fp32-accum",
        "data": "synthetic (seeded, drawn on the GPU)",
        "config": {k: head[k] for k in ("workload", "layers", "batch", "q_heads", "kv_heads", "head_dim",
                                        "cached_tokens", "format", "old_format", "residual", "append_per_step")}
                  | {"parallelism": "none (1 GPU)"},
        "pct_hbm_peak": head["pct_hbm_peak"],
        "decode_steps_per_s": head["steps_per_s"],
        "read_probe_gbs": round(probe, 1),
        "roofline": {"bound": "hbm", "achieved": head["decode_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["decode_frac"], "traffic": traffic_from_profiles(name),
                     "kernel": "decode_kernel (one launch per kvq_append_decode_attn / kvq_decode_attn call)",
                     "launch_us": head["decode_launch_us"], "bytes_per_launch": head["decode_bytes_per_launch"],
                     "timed_launches": args.steps,
                     "read_probe_same_bytes_us": head["read_probe_same_bytes_us"],
                     "decode_vs_read_probe": head["decode_vs_read_probe"]},
    }
    for k in ("prefill_s", "prefill_quantize_ms", "prefill_quantize_gbs", "append_us", "append_note",
              "append_quantize_gbs", "append_quantize_note", "flush_step_ms",
              "plain_step_ms_mean", "flush_append_us", "flush_note", "demote_young", "demotion"):
        if k in head:
            line[k] = head[k]
    model = cpu_model()
    if want_cpu:
        wall, cpu_s, nb, err = head_oracle
        n = len(specs)
        line["cpu_baseline"] = {
            "value": round(nb / wall / 1e9, 4), "unit": "GB/s", "cores": n_workers, "kind": "oracle",
            "cpu_model": model,
            "s_per_step_extrapolated": round(wall / n * head["_pairs_per_step"], 1),
            "sample": f"layer 0, {n} (batch, kv_head) pairs at the final state, each re-quantizing its "
                      f"{head['cached_tokens']} + steps tokens and attending in float64, on {n_workers} worker "
                      f"processes (one BLAS thread each): {wall:.1f} s wall, {cpu_s:.1f} s of worker time; the "
                      f"full step ({head['_pairs_per_step']} pairs) is extrapolated from that rate"}
        line["sample_parity_max_rel_err"] = float(f"{err:.3e}")

    if per_config:
        pc = {}
        jobs = [("c1", None)] + [(w, (st, wu, pairs)) for (w, st, wu, pairs) in PER_CONFIG]
        for w, spec in jobs:
            log(f"per-config {w}")
            if w == "c1":
                r, sp, go = measure_c1()
            else:
                st, wu, pairs = spec
                r, sp, go = measure(w, st, wu, pairs)
            if want_cpu:
                wall, cpu_s, nb, err = run_oracle(pool, sp, go)
                r["parity_max_rel_err"] = float(f"{err:.3e}")
                r["parity_pairs"] = len(sp)
                r["cpu_oracle_s_per_step_extrapolated"] = round(wall / len(sp) * r["_pairs_per_step"], 2)
                r["cpu_oracle_sample"] = (f"layer 0, {len(sp)} pairs in {wall:.2f} s wall on {n_workers} "
                                          f"processes; {r['_pairs_per_step']} pairs per step")
            r.pop("_pairs_per_step", None)
            pc[w] = r
        line["per_config"] = pc
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
