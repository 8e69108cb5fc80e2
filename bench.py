"""Decode-step benchmark of the quantized KV cache on one MI355X.

A step is, for every layer: append one new token (quantize + pack when the fp16 residual is
full, else an fp16 copy into the residual) and one fused dequant + decode-attention call over
the whole cache.  Inputs are seeded synthetic K/V/Q drawn on the GPU before the timed region.

Default workload: 32 layers, batch 8, 32 query / 8 KV heads, head_dim 128, 131072 cached
tokens per sequence in INT4 affine (group 64, fp16 S/Z, 128-token fp16 residual), Student-t
(nu = 4) K and Gaussian V, consecutive decode steps with append and residual flushes.

Output: one JSON line.  `value` is the effective HBM GB/s of the cache read (codes + scales +
zero points + fp16 residual) summed over the timed steps, divided by their wall time.
`roofline` gives the decode-attention call alone, timed with HIP events on the stream it is
launched on.  `cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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


def cpu_baseline(samples, wl, sigma, budget_s: float):
    """Time the CPU oracle on (layer 0, b, kv_head) samples of the final cache state.

    samples: list of (b, h, k chunks, v chunks, q16 [G,128], gpu_out [G,128] fp32); the chunks
    (fp16 [n_i, 128]) are appended in order, as the GPU cache received them.
    Returns (baseline dict, max relative error of the GPU output on the samples)."""
    from threadpoolctl import threadpool_limits
    from oracle.cache import LayerCache
    from oracle.attention import decode_layer
    used = 0
    t_total = 0.0
    bytes_total = 0.0
    worst = 0.0
    with threadpool_limits(limits=1):
        for (b, h, kch, vch, q16, got) in samples:
            t0 = time.perf_counter()
            lc = LayerCache(wl["fmt"], wl["R"], wl["old_fmt"], wl["old_after"], wl.get("demote", False))
            for kc, vc in zip(kch, vch):
                lc.append(kc[None, None], vc[None, None])
            want = decode_layer(lc, q16[None], sigma)[0]
            dt = time.perf_counter() - t0
            t_total += dt
            n_tok = lc.sched.length
            nq_y, nq_o, nr = len(lc.tier_tokens("young")), len(lc.sched.old), len(lc.sched.residual)
            bytes_total += nq_o * bytes_per_token(lc.old_fmt) + nq_y * bytes_per_token(lc.fmt) + nr * 512.0
            worst = max(worst, float(np.abs(got - want).max() / np.abs(want).max()))
            used += 1
            if t_total >= budget_s:
                break
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0, {used} (batch, kv_head) pair(s) x {n_tok} tokens at the final state: "
                      f"quantize every token + fp64 attention of the {samples[0][4].shape[0]} query heads; "
                      f"{t_total:.1f} s on 1 host thread"}, worst


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 64; 320 for c5-demote)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4-int4", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--cpu-pairs", type=int, default=48, help="(batch, kv_head) pairs of layer 0 kept for the oracle")
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

    import torch
    if args.probe == "copy":
        copy_probe()
        return
    if args.study == "noise":
        noise_study([int(x) for x in args.study_lengths.split(",")], args.study_queries)
        return

    import bit_quantized_kv_kvq_amd as kvq
    import kvq_synth as syn

    demote = args.workload in DEMOTE_STEPS
    ragged = args.workload in RAGGED
    if args.steps is None:
        args.steps = DEMOTE_STEPS.get(args.workload, 64)
    cid, fmt_over = WORKLOADS[args.workload]
    W = syn.WORKLOADS[cid]
    fmt = fmt_over or W.fmt
    old_fmt = W.old_fmt or fmt
    L, B, Hq, H, T, R = W.num_layers, W.batch, W.num_q_heads, W.num_kv_heads, W.prefill, W.residual_len
    G = Hq // H
    sigma = 1.0 / np.sqrt(128.0)
    per_step = max(1, W.append_per_step)
    n_steps = args.warmup + args.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    probe = read_probe_gbs()

    cfg = kvq.make_config(L, B, H, T + n_steps * per_step + 1, fmt, R, W.old_fmt, W.old_after, demote=demote)
    cache = kvq.Cache(cfg)
    samples_bh = [(b, h) for b in range(B) for h in range(H)][:args.cpu_pairs]
    host_hist = {bh: ([], []) for bh in samples_bh}

    # ragged: sequence b keeps the first lens[b] of its T drawn tokens
    lens = [T * (b + 1) // B for b in range(B)] if ragged else [T] * B
    if ragged:
        assert W.old_after == 0 and R > 0, "the ragged step tracker models one tier with a residual"

    # ---- untimed state: bulk prefill of every layer (one append of T tokens, or one per
    # sequence when ragged); HIP events around each layer's appends give the bulk quantize rate
    # (fp16 read + packed bytes written)
    t_prefill = time.perf_counter()
    pre_events = []
    for l in range(L):
        k = syn.draw_k_dev(cid, l, B, H, T, W.kdist)
        v = syn.draw_v_dev(cid, l, B, H, T)
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
        if l % 8 == 7 or l == L - 1:
            torch.cuda.synchronize()
            log(f"prefill: {l + 1}/{L} layers, {time.perf_counter() - t_prefill:.1f} s")
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t_prefill
    pre_ms = float(sum(a.elapsed_time(b) for a, b in pre_events))
    pre_bytes = float(L * H * sum(lens) * 2 * 128 * 2) + sum(decode_bytes(cache, l, fmt, old_fmt, ragged)
                                                                for l in range(L))
    # ragged: per (layer, sequence) quantized tokens and residual fill, tracked here (a ctypes
    # query per sequence and layer inside the timed loop would cost host time of its own)
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

    # HIP events around one decode launch per timed step (layer s mod L of step s, so that the
    # sample turns through the layers), created (and each recorded once) before the timed
    # region so that no event set-up falls inside it.  Events around every launch would cost
    # about 3 % of the step time themselves (measured), which the wall clock would then include.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    # and around each append that demotes a block (demotion workloads), likewise made up front
    dem_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(L * (args.steps * per_step // 128 + 2) if demote else 0)]
    for e0, e1 in events + dem_events:
        e0.record(stream)
        e1.record(stream)
    dem_used = []

    def demotes(l):
        """Whether appending this step's tokens to layer l (without a flush) moves a young
        block to the old tier.  The positions stay in order here (one prefill, then steps),
        so the first live young block holds positions [old, old + 128)."""
        if not demote:
            return False
        n_old = cache.layout(l, kvq.REGION_OLD)[2]
        return (cache.layout(l, kvq.REGION_YOUNG)[2] >= 128
                and n_old + 128 <= cache.seq_len(l)[0] + per_step - W.old_after)

    def step(s, ev=None, nbytes=None, timed=None):
        for l in range(L):
            pair = ev if ev is not None and l == timed else None
            # a step whose tokens go straight to the residual is one call and one launch (the
            # copy runs inside the decode launch); a step that quantizes (a full residual, or
            # R = 0) appends first, so that the timed bracket always holds one decode launch
            if ragged:
                quantizes = any(t[1] + per_step > R for t in track[l])
                for t in track[l]:
                    if t[1] + per_step > R:
                        t[0] += t[1] + per_step - ((t[1] + per_step - 1) % R + 1)
                        t[1] = (t[1] + per_step - 1) % R + 1
                    else:
                        t[1] += per_step
            else:
                quantizes = R == 0 or cache.seq_len(l)[1] + per_step > R or demotes(l)
            if args.separate_append or quantizes:
                dem = nbytes is not None and demotes(l) and len(dem_used) < len(dem_events)
                if dem:
                    fb = cache.first_block(l, kvq.REGION_YOUNG)
                    dem_events[len(dem_used)][0].record(stream)
                cache.append(l, knew[s][l], vnew[s][l])
                if dem:
                    dem_events[len(dem_used)][1].record(stream)
                    dem_used.append(cache.first_block(l, kvq.REGION_YOUNG) - fb)
                if pair is not None:
                    pair[0].record(stream)
                cache.decode(l, qs[s][l], sigma, outs[l], ws)
            else:
                if pair is not None:
                    pair[0].record(stream)
                cache.append_decode(l, knew[s][l], vnew[s][l], qs[s][l], sigma, outs[l], ws)
            if pair is not None:
                pair[1].record(stream)
            if nbytes is not None:
                nbytes.append(H * sum(t[0] * bpt + t[1] * 512.0 for t in track[l]) if ragged
                              else decode_bytes(cache, l, fmt, old_fmt))
                if pair is not None:
                    timed_bytes.append(nbytes[-1])

    log("step inputs ready; warmup")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    nbytes, timed_bytes = [], []
    gc.collect()
    gc.disable()            # no collector pause inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, s in enumerate(range(args.warmup, n_steps)):
        step(s, events[i], nbytes, s % L)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    if ragged:   # the tracker agrees with the library's counters
        for l in range(L):
            assert sum(H * (t[0] * bpt + t[1] * 512.0) for t in track[l]) == decode_bytes(cache, l, fmt, old_fmt, True)
    log(f"timed {args.steps} steps in {wall:.3f} s")

    dec_ms = np.array([a.elapsed_time(b) for a, b in events])
    nbytes = np.array(nbytes)
    total_bytes = float(nbytes.sum())
    value = total_bytes / wall / 1e9
    achieved = float(np.mean(timed_bytes) / (dec_ms.mean() * 1e-3) / 1e9)

    # ---- parity on sampled outputs at full size: one more fp32 decode of layer 0
    out32 = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    cache.decode(0, qs[n_steps - 1][0], sigma, out32, ws)
    torch.cuda.synchronize()
    out_h = out32.cpu().numpy().astype(np.float64)
    q_h = qs[n_steps - 1][0].cpu().numpy()
    samples = []
    for (b, h) in samples_bh:
        samples.append((b, h, host_hist[(b, h)][0], host_hist[(b, h)][1], q_h[b, h * G:(h + 1) * G],
                        out_h[b, h * G:(h + 1) * G]))

    line = {
        "metric": "fused dequant+decode-attn effective GB/s (% HBM peak); decode steps/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{fmt}-codes/fp16-operands/fp32-accum",
        "data": "synthetic (seeded, drawn on the GPU)",
        "config": {"workload": (W.name if fmt_over is None else W.name.replace(W.fmt, fmt))
                   + (", young blocks demoted as they age" if demote else "")
                   + (f", ragged: sequence b holds {T}(b+1)/{B} tokens" if ragged else ""),
                   "layers": L, "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": 128,
                   "cached_tokens": lens if ragged else T, "format": fmt, "old_format": W.old_fmt, "residual": R,
                   "append_per_step": per_step, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_steps_per_s": round(args.steps / wall, 2),
        "read_probe_gbs": round(probe, 1),
        "prefill_s": round(t_prefill, 2),
        "prefill_quantize_ms": round(pre_ms, 2),
        "prefill_quantize_gbs": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(args.workload),
                     "kernel": "decode_kernel (one launch per kvq_append_decode_attn / kvq_decode_attn call)",
                     "launch_us": round(float(dec_ms.mean()) * 1e3, 2),
                     "bytes_per_launch": round(float(np.mean(timed_bytes))),
                     "timed_launches": int(dec_ms.size)},
    }
    if demote:
        # each demoted block: one young block read and one old block written per (batch, kv_head)
        blk_bytes = B * H * 128 * (bytes_per_token(fmt) + bytes_per_token(old_fmt))
        dem_ms = np.array([dem_events[i][0].elapsed_time(dem_events[i][1]) for i in range(len(dem_used))])
        nblk = int(sum(dem_used))
        line["config"]["demote_young"] = 1
        line["demotion"] = {"appends": len(dem_used), "blocks": nblk,
                            "append_us": round(float(dem_ms.mean()) * 1e3, 2) if dem_used else None,
                            "bytes_per_block": round(blk_bytes),
                            "gbs": round(blk_bytes * nblk / (dem_ms.sum() * 1e-3) / 1e9, 1) if nblk else None,
                            "note": "event brackets around the whole append call that demotes (its residual "
                                    "copy included)"}
    if not args.no_cpu_baseline:
        wl = {"fmt": fmt, "R": R, "old_fmt": W.old_fmt, "old_after": W.old_after, "demote": demote}
        log("cpu baseline (oracle)")
        base, err = cpu_baseline(samples, wl, sigma, args.cpu_budget)
        line["cpu_baseline"] = base
        line["sample_parity_max_rel_err"] = float(f"{err:.3e}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
