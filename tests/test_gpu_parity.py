"""GPU parity: packed bytes bit-exact and decode attention within 1e-3 * max|out| of the oracle.

Small shapes that span several blocks and a ragged tail; every case names itself in the
test id.  Marked gpu: run on an MI355X."""
import zlib

import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
from gpu_helpers import Pair, adversarial_tokens, assert_attention_close

pytestmark = pytest.mark.gpu

FORMATS = ["int2", "int4", "int8", "nvfp4", "mxfp4", "fp8", "fp16"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [0, 16, 128])
def test_append_bytes_exact(fmt, R):
    rng = np.random.default_rng(zlib.crc32(f"{fmt}/{R}".encode()))
    B, H = 2, 2
    p = Pair(1, B, H, 2000, fmt, R)
    for n in [300, 1, 1, 127, 5, "flush", 129, 1, 250]:
        if n == "flush":
            p.flush(0)
            continue
        p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)


def tie_tokens(rng, B, H, n, qmax, gs):
    """fp16 [B, H, n, 128] whose affine groups of gs dims are built so that x / S is exactly a
    half-integer for most values while 1 / S is not a binary fraction: S = m 2^e (m odd, at
    most 7, so that qmax S is exact), one value at -j S and one at (qmax - j) S fix the group's
    range to qmax S (so S and Z = j come out exactly), the others at (c - j + 1/2) S."""
    ms = [3] if qmax == 255 else [3, 5, 7]
    x = np.empty((B, H, n, 128), np.float64)
    for b in range(B):
        for h in range(H):
            for t in range(n):
                for g0 in range(0, 128, gs):
                    S = float(rng.choice(ms)) * 2.0 ** int(rng.integers(-10, 1))
                    j = int(rng.integers(0, qmax + 1))
                    c = rng.integers(0, qmax, gs)
                    v = (c - j + 0.5) * S
                    pos = rng.permutation(gs)[:2]
                    v[pos[0]], v[pos[1]] = -j * S, (qmax - j) * S
                    x[b, h, t, g0:g0 + gs] = v
    y = x.astype(np.float16)
    assert np.array_equal(y.astype(np.float64), x)
    return y


@pytest.mark.parametrize("fmt", ["int2", "int4", "int8", "int2g32", "int4g32", "int4g128", "int8g128"])
@pytest.mark.parametrize("R", [0, 128])
def test_append_bytes_exact_rounding_ties(fmt, R):
    """Affine codes where x / S is exactly halfway between two codes for most values and S is
    not a power of two: the round-half-even decision of the quantizer, from input and from the
    residual's flush."""
    gs = int(fmt.split("g")[1]) if "g" in fmt else 64
    qmax = (1 << int(fmt[3])) - 1
    rng = np.random.default_rng(zlib.crc32(f"ties/{fmt}/{R}".encode()))
    B, H = 1, 2
    p = Pair(1, B, H, 800, fmt, R)
    for n in [300, 1, 129, 200]:
        p.append(0, tie_tokens(rng, B, H, n, qmax, gs), tie_tokens(rng, B, H, n, qmax, gs))
        p.check_bytes(0)


def test_tiers_bytes_exact():
    rng = np.random.default_rng(77)
    B, H = 1, 2
    p = Pair(1, B, H, 3000, "int4", 128, "int2", 700)
    for n in [1800, 1, 1, 300, "flush", 200]:
        if n == "flush":
            p.flush(0)
            continue
        p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
    assert p.gpu.layout(0, 2)[2] > 0


def test_nvfp4_every_amax():
    """Every positive finite fp16 value as a block maximum (so every E4M3 scale and every
    rounding tie), with the other 15 values drawn below it, plus signed zeros."""
    rng = np.random.default_rng(5)
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = bits.view(np.float16).astype(np.float64)                      # 31743 values
    n_blocks = amax.size
    frac = rng.uniform(-1, 1, (n_blocks, 16))
    x = (frac * amax[:, None]).astype(np.float16)
    x[:, 0] = amax * np.where(rng.random(n_blocks) < 0.5, 1, -1)
    x[::7, 5] = -0.0
    ntok = -(-n_blocks // 8)
    flat = np.zeros((ntok * 8, 16), np.float16)
    flat[:n_blocks] = x
    toks = flat.reshape(1, 1, ntok, 128)
    p = Pair(1, 1, 1, ntok + 8, "nvfp4", 0)
    p.append(0, toks, toks[..., ::-1].copy())
    p.check_bytes(0)


def test_mxfp4_every_amax():
    """Every positive finite fp16 value as the maximum of a 32-value block (so every E8M0 scale
    an fp16 block can have, and the saturating range above 6X), the other 31 values drawn
    below it, plus signed zeros and all-zero blocks."""
    rng = np.random.default_rng(6)
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = bits.view(np.float16).astype(np.float64)
    n_blocks = amax.size + 5
    frac = rng.uniform(-1, 1, (n_blocks, 32))
    frac[:amax.size] *= amax[:, None]
    x = frac.astype(np.float16)
    x[:amax.size, 0] = amax * np.where(rng.random(amax.size) < 0.5, 1, -1)
    x[amax.size:] = 0.0
    x[-1, 3] = -0.0
    x[::7, 5] = -0.0
    ntok = -(-n_blocks // 4)
    flat = np.zeros((ntok * 4, 32), np.float16)
    flat[:n_blocks] = x
    toks = flat.reshape(1, 1, ntok, 128)
    p = Pair(1, 1, 1, ntok + 8, "mxfp4", 0)
    p.append(0, toks, toks[..., ::-1].copy())
    p.check_bytes(0)


def test_fp8_every_fp16_value():
    """Every finite fp16 value (both zeros, subnormals, the rounding ties between E4M3 values,
    the saturating range above 448) through the FP8 cast, as K and (reversed) as V."""
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]                                                 # 63488 values
    rng = np.random.default_rng(8)
    x = x[rng.permutation(x.size)]
    ntok = x.size // 128
    toks = x.reshape(1, 1, ntok, 128)
    p = Pair(1, 1, 1, ntok + 8, "fp8", 0)
    p.append(0, toks, toks[..., ::-1].copy())
    p.check_bytes(0)


@pytest.mark.parametrize("old", ["fp8", "fp16", "mxfp4"])
def test_tier_under_int4(old):
    """FP8 or FP16 as the older tier below an INT4 young tier: bytes of both tiers and the
    decode (one call streams two block formats)."""
    rng = np.random.default_rng(21)
    B, H, G = 1, 2, 4
    p = Pair(1, B, H, 3000, "int4", 128, old, 900)
    for n in [1500, 1, 300, "flush", 77]:
        if n == "flush":
            p.flush(0)
            continue
        p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
    assert p.gpu.layout(0, 2)[2] > 0
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    got, want = p.decode(0, q, 1 / np.sqrt(128))
    assert_attention_close(got, want)


def test_fp16_every_fp16_value():
    """Every finite fp16 value stored bit for bit (signed zeros, subnormals, +-65504)."""
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    x = x[np.random.default_rng(9).permutation(x.size)]
    toks = x.reshape(1, 1, x.size // 128, 128)
    p = Pair(1, 1, 1, x.size // 128 + 8, "fp16", 0)
    p.append(0, toks, toks[..., ::-1].copy())
    p.check_bytes(0)


GROUP_FORMATS = ["int2g32", "int4g32", "int8g32", "int2g128", "int4g128", "int8g128"]


@pytest.mark.parametrize("fmt", GROUP_FORMATS)
def test_group_sizes_bytes_exact(fmt):
    rng = np.random.default_rng(sum(map(ord, fmt)))
    B, H = 2, 2
    p = Pair(1, B, H, 2000, fmt, 128)
    for n in [300, 1, 127, "flush", 129, 250]:
        if n == "flush":
            p.flush(0)
            continue
        p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)


@pytest.mark.parametrize("fmt", GROUP_FORMATS)
@pytest.mark.parametrize("G", [1, 4, 8])
def test_group_sizes_decode(fmt, G):
    rng = np.random.default_rng(G + sum(map(ord, fmt)))
    B, H = 2, 2
    p = Pair(1, B, H, 1400, fmt, 128)
    for L in (129, 1000):
        k = rng.standard_normal((B, H, L, 128)).astype(np.float16)
        k[..., :4] *= 15
        p.append(0, k, rng.standard_normal((B, H, L, 128)).astype(np.float16))
        q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
        for sigma in (1 / np.sqrt(128), 1.0):
            got, want = p.decode(0, q, sigma)
            assert_attention_close(got, want)


def test_debugging_configuration_group32_residual256():
    """The page's debugging configuration: 4 bits, groups of 32, a 256-token residual; flushes
    by filling the residual and explicitly, decode after each."""
    rng = np.random.default_rng(256)
    B, H, G = 2, 2, 4
    p = Pair(1, B, H, 3000, "int4g32", 256)
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    for n in [255, 1, 1, 600, "flush", 3, 300]:
        if n == "flush":
            p.flush(0)
        else:
            p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
        got, want = p.decode(0, q, 1 / np.sqrt(128))
        assert_attention_close(got, want)


KC_FORMATS = ["int2kc", "int4kc", "int8kc"]


@pytest.mark.parametrize("R", [128, 256])
@pytest.mark.parametrize("fmt", KC_FORMATS)
def test_per_channel_k_bytes_and_decode(fmt, R):
    """Per-channel K: windows of 128 tokens flushed from a full residual or quantized in bulk;
    stored bytes and decode (G 1, 4, 8) against the oracle after each append."""
    rng = np.random.default_rng(R + sum(map(ord, fmt)))
    B, H = 2, 2
    p = Pair(1, B, H, 3000, fmt, R)
    for n in [300, 1, 127, 129, 700, 1]:
        k = adversarial_tokens(rng, B, H, n)
        k[..., 7] = np.clip(k[..., 7].astype(np.float32) * 12, -65504, 65504)   # an outlier channel
        p.append(0, k, adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
        for G in (1, 4, 8):
            q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
            got, want = p.decode(0, q, 1 / np.sqrt(128))
            assert_attention_close(got, want)


def test_per_channel_k_tiers_and_partial_flush():
    """Young INT4 and old INT2 tiers both with per-channel K; an explicit flush of a partial
    window is refused and changes nothing."""
    rng = np.random.default_rng(41)
    B, H, G = 1, 2, 4
    p = Pair(1, B, H, 4000, "int4kc", 128, "int2kc", 1000)
    p.append(0, rng.standard_normal((B, H, 2900, 128)).astype(np.float16),
             rng.standard_normal((B, H, 2900, 128)).astype(np.float16))
    p.check_bytes(0)
    assert p.gpu.layout(0, 2)[2] > 0 and p.gpu.seq_len(0)[1] % 128 != 0
    with pytest.raises(kvq.KvqError):
        p.gpu.flush(0)
    p.check_bytes(0)
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    got, want = p.decode(0, q, 1.0)
    assert_attention_close(got, want)


def test_group_size_tiers():
    """Young INT4 and old INT2 tiers sharing groups of 32; adversarial values; decode."""
    rng = np.random.default_rng(31)
    B, H, G = 1, 2, 8
    p = Pair(1, B, H, 3000, "int4g32", 128, "int2g32", 700)
    for n in [1800, 1, 300, "flush", 200]:
        if n == "flush":
            p.flush(0)
            continue
        p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
    assert p.gpu.layout(0, 2)[2] > 0
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    got, want = p.decode(0, q, 1 / np.sqrt(128))
    assert_attention_close(got, want)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("L", [1, 2, 127, 128, 129, 1000])
def test_decode_matches_oracle(fmt, G, L):
    R = 0 if fmt == "nvfp4" else 128
    rng = np.random.default_rng(L * 31 + G)
    B, H = 2, 2
    p = Pair(1, B, H, 1200, fmt, R)
    k = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    k[..., :4] *= 15
    v = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    p.append(0, k, v)
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    for sigma in (1 / np.sqrt(128), 1.0):
        got, want = p.decode(0, q, sigma)
        assert_attention_close(got, want)


@pytest.mark.parametrize("R", [16, 32, 128])
def test_decode_residual_only_and_mixed(R):
    rng = np.random.default_rng(R)
    B, H, G = 1, 3, 4
    p = Pair(1, B, H, 3000, "int4", R)
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    for n in [R // 2, R // 2, 1, 3 * R + 5, "flush", 7]:
        if n == "flush":
            p.flush(0)
        else:
            p.append(0, rng.standard_normal((B, H, n, 128)).astype(np.float16),
                     rng.standard_normal((B, H, n, 128)).astype(np.float16))
        got, want = p.decode(0, q, 1.0)
        assert_attention_close(got, want)


def test_decode_tiers_and_fp16_output():
    rng = np.random.default_rng(3)
    B, H, G = 1, 2, 4
    p = Pair(1, B, H, 4000, "int4", 128, "int2", 1000)
    p.append(0, rng.standard_normal((B, H, 3000, 128)).astype(np.float16),
             rng.standard_normal((B, H, 3000, 128)).astype(np.float16))
    p.append(0, rng.standard_normal((B, H, 1, 128)).astype(np.float16),
             rng.standard_normal((B, H, 1, 128)).astype(np.float16))
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    got, want = p.decode(0, q, 1 / np.sqrt(128))
    assert_attention_close(got, want)
    got16, _ = p.decode(0, q, 1 / np.sqrt(128), out_dtype=torch.float16)
    assert_attention_close(got16, want)


def test_decode_adversarial_values():
    rng = np.random.default_rng(11)
    B, H, G = 1, 2, 8
    for fmt in FORMATS:
        p = Pair(1, B, H, 800, fmt, 0 if fmt == "nvfp4" else 128)
        p.append(0, adversarial_tokens(rng, B, H, 700, 0.5), adversarial_tokens(rng, B, H, 700, 0.5))
        q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
        got, want = p.decode(0, q, 1 / np.sqrt(128))
        assert_attention_close(got, want)


def test_decode_is_deterministic():
    rng = np.random.default_rng(2)
    p = Pair(1, 2, 2, 5000, "int4", 128)
    p.append(0, rng.standard_normal((2, 2, 4500, 128)).astype(np.float16),
             rng.standard_normal((2, 2, 4500, 128)).astype(np.float16))
    q = (rng.standard_normal((2, 8, 128)) / np.sqrt(128)).astype(np.float16)
    outs = [p.decode(0, q, 1.0)[0] for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("fmt", FORMATS)
def test_decode_rotated_block_order_with_partial_block(fmt):
    """Each (batch, kv_head) visits its blocks rotated by a hashed offset; with 38 blocks (37
    full, the last holding 5 slots) the four (b, h) get rotations 0, 25, 6 and 31, which wrap
    past the partial block, and it must still be the one whose tail slots are masked.  Every
    token is quantized (residual 0), so every format has the partial block."""
    rng = np.random.default_rng(zlib.crc32(f"rot/{fmt}".encode()))
    B, H, G, L = 2, 2, 4, 37 * 128 + 5
    p = Pair(1, B, H, L + 64, fmt, 0)
    k = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    k[..., :4] *= 15
    v = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    p.append(0, k, v)
    assert p.gpu.layout(0, 1)[2] == L and L % 128 == 5       # 37 full blocks and a partial one
    p.check_bytes(0)
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    for sigma in (1 / np.sqrt(128), 1.0):
        got, want = p.decode(0, q, sigma)
        assert_attention_close(got, want)


@pytest.mark.parametrize("fmt", ["int4", "nvfp4", "fp16"])
@pytest.mark.parametrize("G", [2, 3, 6, 12, 16])
@pytest.mark.parametrize("L", [700, 20000])
def test_decode_other_group_sizes(fmt, G, L):
    """Query heads per kv head other than 1, 4 and 8 (the merge splits the G * 32 output
    columns over thread groups, or gives a thread two of them at G = 16), with few and with
    many work items per (batch, kv_head): 20000 tokens of 2 kv heads give 128 items each."""
    rng = np.random.default_rng(zlib.crc32(f"og/{fmt}/{G}/{L}".encode()))
    B, H = 1, 2
    R = 0 if fmt == "nvfp4" else 128
    p = Pair(1, B, H, L + 8, fmt, R)
    k = rng.standard_normal((B, H, L, 128)).astype(np.float16)
    k[..., :4] *= 15
    p.append(0, k, rng.standard_normal((B, H, L, 128)).astype(np.float16))
    q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
    for sigma in (1 / np.sqrt(128), 1.0):
        got, want = p.decode(0, q, sigma)
        assert_attention_close(got, want)
