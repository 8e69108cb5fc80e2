"""Pins of the residual / tier schedule: closed-form counts and bulk == one-by-one."""
import numpy as np
import pytest

from oracle.cache import Schedule, LayerCache


@pytest.mark.parametrize("L", [1, 2, 127, 128, 129, 255, 256, 257, 1000, 1152])
def test_counts_from_empty(L):
    s = Schedule(128)
    s.append(L)
    nq = 128 * ((L - 1) // 128)
    assert len(s.young) == nq and len(s.residual) == L - nq and 1 <= len(s.residual) <= 128
    assert s.young == list(range(nq)) and s.residual == list(range(nq, L))


def test_single_token_steps_127_128_129():
    s = Schedule(128)
    for L in range(1, 130):
        s.append(1)
        if L == 128:
            assert len(s.residual) == 128 and not s.young        # lazy: full but not flushed
        if L == 129:
            assert len(s.young) == 128 and s.residual == [128] and s.flushes == 1


def test_workload_states():
    s = Schedule(128); s.append(1152)
    assert (len(s.young), len(s.residual)) == (1024, 128)           # 1K int4 + 128 fp16
    s = Schedule(128); s.append(1024)
    assert (len(s.young), len(s.residual)) == (896, 128)
    s.append(128)
    assert (len(s.young), len(s.residual), s.flushes) == (1024, 128, 8)   # exactly one flush in the append
    s = Schedule(128, old_after=65536); s.append(262144)
    assert (len(s.old), len(s.young), len(s.residual)) == (196608, 65408, 128)
    assert s.old == list(range(196608))
    s.append(1)                                                      # next step flushes into the young tier
    assert (len(s.old), len(s.young), len(s.residual)) == (196608, 65536, 1)
    s = Schedule(0); s.append(32768)
    assert (len(s.young), len(s.residual)) == (32768, 0)


def test_explicit_flush():
    s = Schedule(128); s.append(200); s.flush()
    assert len(s.young) == 200 and not s.residual
    s.flush()
    assert len(s.young) == 200
    s.append(5)
    assert s.residual == [200, 201, 202, 203, 204]


@pytest.mark.parametrize("fmt,R,old_after", [("int4", 128, 0), ("int2", 16, 0), ("nvfp4", 0, 0),
                                             ("int4", 32, 100), ("int8", 128, 0)])
def test_bulk_equals_one_by_one(fmt, R, old_after):
    """Appending n tokens at once stores the same bytes as appending them one at a time,
    except where a tier decision depends on the call boundary (old_after > 0)."""
    rng = np.random.default_rng(1)
    n = 300
    k = rng.standard_normal((1, 2, n, 128)).astype(np.float16)
    v = rng.standard_normal((1, 2, n, 128)).astype(np.float16)
    a = LayerCache(fmt, R, "int2" if old_after else None, old_after)
    a.append(k[:, :, :50], v[:, :, :50]); a.append(k[:, :, 50:], v[:, :, 50:])
    b = LayerCache(fmt, R, "int2" if old_after else None, old_after)
    for t in range(n):
        b.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
    if old_after:
        # one-by-one never makes a token old-tier before it is old_after behind; bulk may
        assert len(b.sched.old) <= len(a.sched.old)
        return
    for h in range(2):
        assert np.array_equal(a.arena(0, h, "young"), b.arena(0, h, "young"))
        ra, rb = a.residual(0, h), b.residual(0, h)
        assert np.array_equal(ra[0][ra[1]], rb[0][rb[1]])


def test_demotion_moves_whole_aged_blocks():
    """With demotion, every full young block whose last token falls old_after behind moves to
    the old tier at the end of the append (closed form for one-token appends after a prefill)."""
    from oracle.cache import Schedule
    s = Schedule(128, old_after=1000, demote=True)
    s.append(900)                                  # all young: nothing is 1000 behind
    assert s.old == [] and s.live_young() == list(range(896))     # 7 flushed chunks; 4 in the residual
    s.append(400)                                  # L = 1300: blocks ending at <= 300 demote
    assert s.old == list(range(256)) and all(s.old_demoted)
    assert s.live_young()[0] == 256
    for _ in range(1000):                          # one token at a time
        s.append(1)
    L = 2300
    # every full young block whose last position + 1 <= L - 1000 has moved, in order
    assert s.old == list(range(len(s.old))) and len(s.old) % 128 == 0
    assert len(s.old) == ((L - 1000) // 128) * 128
    assert s.live_young()[0] == len(s.old)
    # tokens are conserved and no position is in two places
    allpos = s.old + s.live_young() + s.residual
    assert sorted(allpos) == list(range(L))


def test_demotion_off_and_static_tiers_unchanged():
    from oracle.cache import Schedule
    a, b = Schedule(128, old_after=500), Schedule(128, old_after=500, demote=False)
    for n in [600, 1, 1, 300, 700]:
        a.append(n); b.append(n)
    assert a.old == b.old and a.young == b.young and not any(a.old_demoted)


def test_demoted_tokens_are_requantized_from_young_values():
    """The old tier's demoted slots decode to the old format applied to the fp16 rounding of the
    young decoded values (not of the original inputs)."""
    import numpy as np
    from oracle.cache import LayerCache
    from oracle.quant import quantize_tokens, dequantize_tokens
    rng = np.random.default_rng(3)
    c = LayerCache("int4", 128, "int2", 300, demote=True)
    k = rng.standard_normal((1, 1, 800, 128)).astype(np.float16)
    c.append(k, k)
    c.append(k[:, :, :100], k[:, :, :100])
    assert any(c.sched.old_demoted)
    ki, _ = c.tier_inputs(0, 0, "old")
    pos = np.asarray(c.sched.old)
    dem = np.asarray(c.sched.old_demoted)
    # 384 tokens went old directly (static rule), then the young block 384..511 was demoted
    assert list(pos) == list(range(512)) and not dem[:384].any() and dem[384:].all()
    young_hat = dequantize_tokens(quantize_tokens(k[0, 0][pos[dem]], "int4"), "int4")
    assert np.array_equal(ki[dem].astype(np.float64), young_hat.astype(np.float16).astype(np.float64))
    assert np.array_equal(ki[~dem], k[0, 0][pos[~dem]])
    assert not np.array_equal(ki[dem], k[0, 0][pos[dem]])
