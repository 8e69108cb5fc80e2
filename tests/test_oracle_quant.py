"""Pins of the oracle's affine and NVFP4 quantizers: brute-force nearest codes, exact
rational S and Z, and the invariants the method implies."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, numerics as nm


def _groups(seed, n=400, w=64):
    """Random and adversarial fp16 groups of w values."""
    r = np.random.default_rng(seed)
    gs = [r.standard_normal((n, w)),
          r.standard_normal((n // 4, w)) * 15.0,
          r.standard_t(4, (n // 4, w)),
          r.uniform(3.0, 3.01, (n // 8, w)),            # narrow, not straddling 0
          -r.uniform(100, 101, (n // 8, w)),
          r.standard_normal((n // 8, w)) * 1e-6,       # subnormal territory
          np.clip(r.standard_normal((n // 8, w)) * 40000, -65504, 65504)]
    two = np.where(r.random((n // 8, w)) < 0.5, -1.25, 2.5); two[:, 0] = -1.25; two[:, 1] = 2.5
    gs.append(two)
    ties = np.round(r.standard_normal((n // 8, w)) * 8) / 2   # many half-integers
    gs.append(ties)
    return np.concatenate(gs).astype(np.float16)


@pytest.mark.parametrize("w", [32, 64, 128])
@pytest.mark.parametrize("nbits", [2, 4, 8])
def test_codes_are_brute_force_nearest(nbits, w):
    """Each code is the nearest valid code: argmin over q in [0, 2^n-1] of |x - S(q - Z)|,
    ties broken towards even q - Z (round half to even of x/S)."""
    g = _groups(nbits, w=w)
    q, S, Z = quant.affine_quantize(g, nbits)
    qmax = (1 << nbits) - 1
    cand = np.arange(qmax + 1, dtype=np.float64)
    dec = S.astype(np.float64)[:, None] * (cand[None, :] - Z.astype(np.float64)[:, None])   # [G, 2^n]
    x = g.astype(np.float64)
    dist = np.abs(x[:, :, None] - dec[:, None, :])                   # exact in float64
    best = dist.min(axis=2, keepdims=True)
    tied = dist == best
    even = tied & (((cand[None, None, :] - Z.astype(np.float64)[:, None, None]) % 2) == 0)
    expect = np.where(tied.sum(axis=2) > 1, np.argmax(even, axis=2), np.argmax(tied, axis=2))
    assert np.array_equal(q.astype(np.int64), expect)


@pytest.mark.parametrize("w", [32, 64, 128])
@pytest.mark.parametrize("nbits", [2, 4, 8])
def test_scale_and_zero_exact_rational(nbits, w):
    g = _groups(10 + nbits, 200, w)
    q, S, Z = quant.affine_quantize(g, nbits)
    qmax = (1 << nbits) - 1
    for row, s, z in zip(g, S, Z):
        mn, mx = Fraction(float(row.min())), Fraction(float(row.max()))
        t = (mx - mn) / qmax
        s_exact_nearest = None
        if mx > mn:
            lo = np.float16(float(t))
            cands = [c for c in {lo, np.nextafter(lo, np.float16(np.inf)), np.nextafter(lo, np.float16(0))}]
            best = min(abs(Fraction(float(c)) - t) for c in cands)
            tied = [c for c in cands if abs(Fraction(float(c)) - t) == best]
            if len(tied) > 1:
                tied = [c for c in tied if (np.array(c, np.float16).view(np.uint16) & 1) == 0]
            s_exact_nearest = float(tied[0])
        if s_exact_nearest:
            assert float(s) == s_exact_nearest
        else:                                   # degenerate: S = |min|, or 1 when min is 0
            assert float(s) == (abs(float(mn)) if mn != 0 else 1.0)
        zq = -mn / Fraction(float(s))
        zi = int(zq.__round__())                # Fraction.__round__ rounds half to even
        zi = max(-65504, min(65504, zi))
        assert float(z) == float(np.float16(zi)), (float(mn), float(s), zi)


@pytest.mark.parametrize("w", [32, 64, 128])
@pytest.mark.parametrize("nbits", [2, 4, 8])
def test_invariants(nbits, w):
    g = _groups(20 + nbits, w=w)
    q, S, Z = quant.affine_quantize(g, nbits)
    qmax = (1 << nbits) - 1
    x = g.astype(np.float64)
    xh = quant.affine_dequantize(q, S, Z)
    S64 = S.astype(np.float64)[:, None]
    small_z = np.abs(Z.astype(np.float64)) <= 2048
    # (i) the minimum of a group always gets code 0 (when Z is stored exactly)
    amin = np.argmin(x, axis=1)
    assert np.all(q[np.arange(len(q)), amin][small_z] == 0)
    # (ii) round-trip error <= S/2 for values whose code is not clamped
    raw = np.rint(x / S64) + Z.astype(np.float64)[:, None]
    unclamped = (raw >= 0) & (raw <= qmax)
    assert np.all(np.abs(x - xh)[unclamped] <= 0.5 * np.broadcast_to(S64, x.shape)[unclamped])
    # (iii) projection: quantizing the decoded values with the same (S, Z) gives q back
    q2 = np.clip(np.rint(xh / S64) + Z.astype(np.float64)[:, None], 0, qmax)
    assert np.array_equal(q2, q.astype(np.float64))
    # (iv) idempotence: re-quantizing the decoded group from scratch reproduces (S, Z, q)
    #      when the group's codes span [0, 2^n - 1] and x_hat is representable in fp16
    span = (q.min(axis=1) == 0) & (q.max(axis=1) == qmax)
    with np.errstate(over="ignore"):
        rep = np.all(xh.astype(np.float16).astype(np.float64) == xh, axis=1)
    sel = span & rep & small_z
    # int8 decoded values rarely fit fp16 (11 significant bits), so few groups qualify
    assert sel.sum() > (100 if nbits <= 4 else 0)
    q3, S3, Z3 = quant.affine_quantize(xh[sel].astype(np.float16), nbits)
    assert np.array_equal(q3, q[sel]) and np.array_equal(S3, S[sel]) and np.array_equal(Z3, Z[sel])


def test_constant_and_two_valued_groups():
    for c in [0.0, -0.0, 1.5, -7.25, 65504.0, 2.0 ** -24]:
        g = np.full((1, 64), c, np.float16)
        for nb in (2, 4, 8):
            q, S, Z = quant.affine_quantize(g, nb)
            assert np.array_equal(quant.affine_dequantize(q, S, Z), g.astype(np.float64))
            assert np.all(q == 0)
    g = np.where(np.arange(64) % 3 == 0, -2.0, 5.0).astype(np.float16)[None]
    for nb in (2, 4, 8):
        q, S, Z = quant.affine_quantize(g, nb)
        assert set(np.unique(q)) == {0, (1 << nb) - 1}


def test_zero_is_stored_as_positive_zero():
    g = np.zeros((2, 64), np.float16); g[1, :] = -0.0
    g[0, 5] = 1.0
    _, _, Z = quant.affine_quantize(g, 4)
    assert np.all(Z.view(np.uint16) == 0)


def test_nvfp4_block_quantizer():
    r = np.random.default_rng(3)
    x = (r.standard_normal((500, 16)) * np.exp2(r.integers(-12, 10, (500, 1)))).astype(np.float16)
    codes, sb = quant.nvfp4_quantize(x)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    assert np.array_equal(sb, nm.e4m3_encode(amax / 6))
    s = nm.e4m3_decode(sb)
    xh = quant.nvfp4_dequantize(codes, sb)
    # decoded magnitudes never exceed 6 * s, and each element is the nearest grid value
    assert np.all(np.abs(xh) <= 6 * s[:, None])
    grid = np.asarray(nm.E2M1_MAGNITUDES)[None, None, :] * s[:, None, None]
    d_best = np.abs(np.abs(x.astype(np.float64))[:, :, None] - grid).min(axis=2)
    assert np.array_equal(np.abs(np.abs(x.astype(np.float64)) - np.abs(xh)), d_best)
    # an all-zero block has scale 0 and signed-zero codes
    z = np.array([[0.0] * 8 + [-0.0] * 8], np.float16)
    c0, s0 = quant.nvfp4_quantize(z)
    assert s0[0] == 0 and list(c0[0]) == [0] * 8 + [8] * 8
    # a block whose amax/6 exceeds 448 saturates the scale
    big = np.full((1, 16), 60000.0, np.float16)
    _, sbig = quant.nvfp4_quantize(big)
    assert sbig[0] == 0x7E


def test_fp16_format_stores_the_values_themselves():
    """The unquantized format keeps every finite fp16 value bit for bit (signed zeros and
    subnormals included) and decodes it exactly."""
    from oracle.quant import quantize_tokens, dequantize_tokens
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)][:63488 // 128 * 128].reshape(-1, 128)
    q = quantize_tokens(x, "fp16")
    assert np.array_equal(q["codes"], x.view(np.uint16))
    xh = dequantize_tokens(q, "fp16")
    assert np.array_equal(xh, x.astype(np.float64))
    assert np.array_equal(np.signbit(xh), np.signbit(x))


def test_mx_scale_exhaustive_over_fp16_amax():
    """For every positive finite fp16 block maximum the E8M0 scale X is the power of two with
    4 <= amax / X < 8 (the largest magnitude then lands in E2M1's top binade [4, 8))."""
    from oracle.quant import mxfp4_quantize
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = bits.view(np.float16)
    x = np.zeros((amax.size, 32), np.float16)
    x[:, 7] = amax
    x[::2, 7] *= -1                                  # the sign does not matter
    _, sb = mxfp4_quantize(x)
    X = np.ldexp(1.0, sb.astype(np.int64) - 127)
    r = amax.astype(np.float64) / X
    assert np.all((r >= 4) & (r < 8))
    assert sb.min() == 127 - 26 and sb.max() == 127 + 13    # 2^-24 and 65504


def test_mxfp4_codes_brute_force():
    """Each code is the E2M1 magnitude nearest to min(|x| / X, 6) (ties to the even code), with
    x's sign bit; decoding multiplies by X exactly."""
    from oracle.quant import mxfp4_quantize, mxfp4_dequantize
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((4000, 32)) * np.exp2(rng.integers(-20, 12, (4000, 1)))).astype(np.float16)
    x[::5] = np.round(x[::5].astype(np.float64) * 4) / 4            # many exact grid points and ties
    x[3::7, 2] = -0.0
    codes, sb = mxfp4_quantize(x)
    X = np.ldexp(1.0, sb.astype(np.int64) - 127)[:, None]
    t = np.minimum(np.abs(x.astype(np.float64)) / X, 6.0)
    d = np.abs(t[..., None] - mags)                                  # [n, 32, 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # nearest; on a tie the even index
    want = np.where(cand.sum(-1) > 1, np.argmax(cand & (np.arange(8) % 2 == 0), axis=-1), np.argmax(cand, axis=-1))
    assert np.array_equal(codes & 7, want)
    assert np.array_equal(codes >> 3, np.signbit(x).astype(np.uint8))
    xh = mxfp4_dequantize(codes, sb)
    assert np.array_equal(xh, np.where(codes & 8, -1, 1) * mags[codes & 7] * X)


def test_mxfp4_saturation_and_zero_block():
    """Values between 6X and 8X saturate to 6X (amax = 7 * 2^k gives X = 2^(k+0), since
    floor(log2 7) = 2); an all-zero block stores the smallest scale and signed zeros."""
    from oracle.quant import mxfp4_quantize, mxfp4_dequantize
    x = np.zeros((2, 32), np.float16)
    x[0, 0] = 7.0
    x[0, 1] = -3.0
    x[1, 5] = -0.0
    codes, sb = mxfp4_quantize(x)
    assert sb[0] == 127 and codes[0, 0] == 7 and codes[0, 1] == 8 + 5
    assert mxfp4_dequantize(codes, sb)[0, 0] == 6.0
    assert sb[1] == 0 and codes[1, 5] == 8 and not codes[1, :5].any()


@pytest.mark.parametrize("fmt", ["int4g32", "int2g32", "int8g128", "int4"])
def test_token_groups_are_contiguous_head_dim_runs(fmt):
    """quantize_tokens splits each token's 128 values into 128/g runs of g contiguous dims."""
    n, gs = quant.affine_params(fmt)
    x = _groups(5, 64, 128)
    qt = quant.quantize_tokens(x, fmt)
    assert qt["S"].shape == (x.shape[0], 128 // gs)
    for G in range(128 // gs):
        q, S, Z = quant.affine_quantize(x[:, gs * G:gs * (G + 1)], n)
        assert np.array_equal(qt["codes"][:, gs * G:gs * (G + 1)], q)
        assert np.array_equal(qt["S"][:, G], S) and np.array_equal(qt["Z"][:, G], Z)


def test_affine_format_names():
    assert quant.affine_params("int4") == (4, 64)
    assert quant.affine_params("int2g32") == (2, 32)
    assert quant.affine_params("int8g128") == (8, 128)
    for bad in ("int3", "int4g16", "nvfp4", "fp8", "int4g"):
        assert quant.affine_params(bad) is None


@pytest.mark.parametrize("fmt", ["int4kc", "int2kc", "int8kc"])
def test_per_channel_k_groups_are_dims_of_a_window(fmt):
    """K: each dim's values over a window of 128 consecutive tokens are one affine group; V
    is quantized per token exactly as the groups-of-64 format."""
    n = quant.affine_params(fmt)[0]
    x = _groups(7, 128, 128)[:256]                      # two windows of 128 tokens
    x[:, 9] = np.clip(x[:, 9].astype(np.float64) * 40, -65504, 65504).astype(np.float16)   # an outlier channel
    qk = quant.quantize_tokens(x, fmt, "k")
    assert qk["S"].shape == (2, 128)
    for w in range(2):
        win = x[128 * w:128 * (w + 1)]
        q, S, Z = quant.affine_quantize(np.ascontiguousarray(win.T), n)      # rows = dims
        assert np.array_equal(qk["codes"][128 * w:128 * (w + 1)], q.T)
        assert np.array_equal(qk["S"][w], S) and np.array_equal(qk["Z"][w], Z)
    xh = quant.dequantize_tokens(qk, fmt, "k")
    assert np.array_equal(xh[:128, 9], quant.affine_dequantize(qk["codes"][:128, 9][None], qk["S"][0, 9:10], qk["Z"][0, 9:10])[0])
    qv, qv64 = quant.quantize_tokens(x, fmt, "v"), quant.quantize_tokens(x, f"int{n}")
    assert all(np.array_equal(qv[k], qv64[k]) for k in qv64)
    with pytest.raises(AssertionError):
        quant.quantize_tokens(x[:100], fmt, "k")
