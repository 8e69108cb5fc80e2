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
