"""GPU: the decode work split and its workspace.

* The workspace's contents on entry do not matter (zeros, all ones, random bytes).
* One workspace serves several caches and shapes in turn (counters are tagged per call).
* The deterministic split (chunks assigned up front) is bitwise reproducible; the default
  split (chunks handed out through the cursor) stays within the attention tolerance.

One (batch, kv_head) pair with 262,221 INT4 tokens is large enough (2048 blocks for 128 work
items) that the default split hands chunks out through the cursor; a two-tier pair of 300K
tokens (two tiers of about 1171 blocks, 64 items each) exercises one cursor per tier; a
100K-token pair, whose blocks are dealt round-robin, changes length between calls."""
import numpy as np
import pytest
import torch

from gpu_helpers import Pair, assert_attention_close, to_dev
from oracle.attention import decode_layer

pytestmark = pytest.mark.gpu

SIGMA = 1 / np.sqrt(128)


def _pair(T, G, seed, fmt="int4", old_fmt=None, old_after=0):
    rng = np.random.default_rng(seed)
    p = Pair(1, 1, 1, T + 8, fmt, 128, old_fmt, old_after)
    k = rng.standard_normal((1, 1, T, 128)).astype(np.float16)
    k[..., :4] *= 15
    v = rng.standard_normal((1, 1, T, 128)).astype(np.float16)
    p.append(0, k, v)
    q = (rng.standard_normal((1, G, 128)) / np.sqrt(128)).astype(np.float16)
    return p, q


def _decode(p, q16, ws):
    out = torch.empty((1, q16.shape[1], 128), dtype=torch.float32, device="cuda")
    p.gpu.decode(0, to_dev(q16), SIGMA, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def big():
    p, q = _pair(262144 + 77, 4, 1)
    return p, q, decode_layer(p.ora[0], q, SIGMA)


def _workspace(p, Hq, fill):
    ws = torch.empty(p.gpu.workspace_bytes(Hq), dtype=torch.uint8, device="cuda")
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(255)
    else:
        g = torch.Generator(device="cuda").manual_seed(fill)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    return ws


@pytest.mark.parametrize("fill", ["zeros", "ones", 7, 8])
def test_workspace_contents_do_not_matter(big, fill):
    p, q, want = big
    ws = _workspace(p, q.shape[1], fill)
    for _ in range(3):                      # later calls find the words this call tagged
        assert_attention_close(_decode(p, q, ws), want)


def test_deterministic_split_is_bitwise_reproducible(big):
    p, q, want = big
    p.gpu.set_deterministic(True)
    try:
        outs = [_decode(p, q, _workspace(p, q.shape[1], fill)) for fill in ("zeros", "ones", 3, "zeros")]
    finally:
        p.gpu.set_deterministic(False)
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert_attention_close(outs[0], want)
    # the default split (other summation order and running maxima) meets the same bar
    assert_attention_close(_decode(p, q, _workspace(p, q.shape[1], "zeros")), want)


def test_one_workspace_for_several_caches(big):
    """Calls on different caches and shapes alternate on one workspace; each must find only
    its own call's counters."""
    p1, q1, want1 = big
    p2, q2 = _pair(300000 + 5, 8, 2, "int4", "int2", 150000)     # two tiers: two cursors per pair
    want2 = decode_layer(p2.ora[0], q2, SIGMA)
    p3, q3 = _pair(3000, 1, 3)                                     # small: chunks dealt round-robin
    want3 = decode_layer(p3.ora[0], q3, SIGMA)
    nbytes = max(p.gpu.workspace_bytes(q.shape[1]) for p, q in ((p1, q1), (p2, q2), (p3, q3)))
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        for p, q, want in ((p1, q1, want1), (p2, q2, want2), (p3, q3, want3), (p2, q2, want2)):
            assert_attention_close(_decode(p, q, ws), want)


def test_append_between_calls_on_one_workspace():
    """Decode, append one token, decode again: the lengths (and so the split) change between
    calls that share the workspace."""
    p, q = _pair(100000 + 127, 4, 4)
    ws = _workspace(p, 4, 11)
    rng = np.random.default_rng(9)
    for _ in range(3):
        assert_attention_close(_decode(p, q, ws), decode_layer(p.ora[0], q, SIGMA))
        p.append(0, rng.standard_normal((1, 1, 1, 128)).astype(np.float16),
                 rng.standard_normal((1, 1, 1, 128)).astype(np.float16))
