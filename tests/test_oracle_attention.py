"""Pins of the oracle's attention: brute force in 50-digit decimal, torch SDPA on a
residual-only cache, and closed forms."""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle.attention import attend, decode_layer
from oracle.cache import LayerCache


def test_brute_force_decimal():
    getcontext().prec = 50
    rng = np.random.default_rng(5)
    for T in range(1, 9):
        q = rng.standard_normal((2, 4)).astype(np.float16)
        k = rng.standard_normal((T, 4)) * 3
        v = rng.standard_normal((T, 4))
        sigma = 0.7
        out = attend(q, k, v, sigma)
        for g in range(2):
            s = [Decimal(sigma) * sum(Decimal(float(q[g, d])) * Decimal(k[t, d]) for d in range(4)) for t in range(T)]
            e = [x.exp() for x in s]
            z = sum(e)
            for d in range(4):
                ref = sum(e[t] / z * Decimal(v[t, d]) for t in range(T))
                assert abs(float(ref) - out[g, d]) <= 1e-12 * max(1.0, abs(float(ref)))


@pytest.mark.parametrize("sigma", [1 / np.sqrt(128), 1.0])
def test_residual_only_cache_is_plain_sdpa(sigma):
    """With fewer than R tokens nothing is quantized: the layer reduces to textbook SDPA."""
    rng = np.random.default_rng(9)
    B, H, G, L = 2, 2, 4, 100
    k = (rng.standard_normal((B, H, L, 128)) * 2).astype(np.float16)
    v = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float16)
    c = LayerCache("int4", 128)
    c.append(k, v)
    out = decode_layer(c, q, sigma)
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(sigma))[:, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((50, 128)); v = rng.standard_normal((50, 128))
    # q = 0: uniform weights, the mean of v
    assert np.allclose(attend(np.zeros((1, 128)), k, v, 1.0), v.mean(axis=0), atol=1e-13)
    # one token: its value
    assert np.allclose(attend(rng.standard_normal((3, 128)), k[:1], v[:1], 1.0), np.repeat(v[:1], 3, 0), atol=1e-13)
    # identical queries give identical outputs; permuting tokens changes nothing
    q = np.repeat(rng.standard_normal((1, 128)), 4, 0)
    o = attend(q, k, v, 0.3)
    assert np.all(o == o[0])
    p = rng.permutation(50)
    assert np.allclose(attend(q, k[p], v[p], 0.3), o, atol=1e-13)
    # one dominant key with a large scale: output -> that key's value
    kd = k.copy(); kd[17] = 50 * q[0] / np.linalg.norm(q[0])
    assert np.allclose(attend(q[:1], kd, v, 10.0), v[17], atol=1e-9)
