"""GPU: a decode call captured in a HIP graph and replayed.

A call's device work is fixed when it is enqueued (its lengths, split and call tag are kernel
arguments), and each launch leaves its arrival counters and chunk cursors at zero when it ends,
so a captured kvq_decode_attn replays the same attention each time.  The graph is replayed
several times, with eager library calls, other device work and host synchronizations between
the replays, and with new query values written into the captured query buffer before each
replay; every replay must equal (bitwise: deterministic split) an eager call on the same query.
"""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,R,n", [("int4", 128, 3000), ("int2", 128, 2500), ("nvfp4", 0, 2048)])
def test_captured_decode_replays_match_eager(fmt, R, n):
    torch.cuda.set_device(0)
    B, H, G = 2, 4, 4
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    cache = kvq.Cache(kvq.make_config(1, B, H, n + 16, fmt, R))
    k = torch.randn((B, H, n, 128), generator=g, device="cuda").half()
    v = torch.randn((B, H, n, 128), generator=g, device="cuda").half()
    cache.append(0, k, v)
    cache.set_deterministic(True)
    ws = torch.empty(cache.workspace_bytes(H * G), dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty_like(ws)
    q = torch.randn((B, H * G, 128), generator=g, device="cuda").half()
    out_g = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)
    scale = 1.0 / np.sqrt(128.0)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cache.decode(0, q, scale, out_g, ws)          # first call outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cache.decode(0, q, scale, out_g, ws)
    torch.cuda.synchronize()

    for r in range(4):
        q.copy_(torch.randn((B, H * G, 128), generator=g, device="cuda").half())
        cache.decode(0, q, scale, out_e, ws_eager)     # eager reference on the same query
        torch.cuda.synchronize()
        junk = torch.randn((1 << 20,), device="cuda").sum()   # other device work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out_g, out_e), f"replay {r}: max |diff| {(out_g - out_e).abs().max().item():.3e}"
        print(f"{fmt}: replay {r} equals the eager call (max|out| {out_e.abs().max().item():.3f})")
