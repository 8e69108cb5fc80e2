"""kvq_decode_attn_noalloc (workspace in the library's per-GPU scratch array) against
kvq_decode_attn (caller's workspace) on the same cache: two calls in a row, the second on a
smaller input, then the first shape again; bitwise equal with the deterministic split, and
within the attention tolerance of the oracle with the default (cursor) split."""
import numpy as np
import pytest
import torch

from gpu_helpers import Pair, assert_attention_close, to_dev

pytestmark = pytest.mark.gpu

CASES = [(4, 8, 4, 5000, "int4", 128), (1, 2, 8, 700, "nvfp4", 0), (4, 8, 4, 5000, "int4", 128)]


def _pair(B, H, L, fmt, R, seed):
    rng = np.random.default_rng(seed)
    p = Pair(1, B, H, L + 8, fmt, R)
    p.append(0, rng.standard_normal((B, H, L, 128)).astype(np.float16),
             rng.standard_normal((B, H, L, 128)).astype(np.float16))
    return p, rng


@pytest.mark.parametrize("deterministic", [True, False])
def test_noalloc_matches_decode_attn(deterministic):
    for i, (B, H, G, L, fmt, R) in enumerate(CASES):
        p, rng = _pair(B, H, L, fmt, R, 100 + i)
        p.gpu.set_deterministic(deterministic)
        q16 = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
        q = to_dev(q16)
        ws = torch.empty(p.gpu.workspace_bytes(H * G), dtype=torch.uint8, device="cuda")
        ref = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
        got = torch.empty_like(ref)
        p.gpu.decode(0, q, 1 / np.sqrt(128), ref, ws)
        p.gpu.decode_noalloc(0, q, 1 / np.sqrt(128), got)
        torch.cuda.synchronize()
        a, b = got.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)
        if deterministic:
            assert np.array_equal(a, b), f"case {i}: no-alloc output differs from kvq_decode_attn's"
        else:
            assert_attention_close(a, b)
        _, want = p.decode(0, q16, 1 / np.sqrt(128))
        assert_attention_close(a, want)
