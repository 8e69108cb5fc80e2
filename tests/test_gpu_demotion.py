"""GPU: age-based demotion (young blocks re-quantized into the old tier as tokens age, page
"KV缓存量化技术：提升大模型长文本生成效率" §4.2).  The stored bytes of both tiers (the
young tier from its first live block) and the residual equal the oracle's after every
append and flush, and the decode of the mixed cache is within the attention tolerance."""
import numpy as np
import pytest

from gpu_helpers import Pair, adversarial_tokens, assert_attention_close

pytestmark = pytest.mark.gpu

SIGMA = 1 / np.sqrt(128)


@pytest.mark.parametrize("fmt,R,old,old_after", [("int4", 128, "int2", 300), ("int8", 0, "nvfp4", 200),
                                                  ("int2", 16, "mxfp4", 129), ("int4", 256, "fp8", 64),
                                                  ("int8", 128, "int4", 128), ("int4", 128, "int8", 500)])
def test_demotion_bytes_and_decode(fmt, R, old, old_after):
    rng = np.random.default_rng(old_after)
    B, H, G = 2, 2, 4
    p = Pair(1, B, H, 4000, fmt, R, old, old_after, demote=True)
    for step, n in enumerate([700, 1, 1, 130, "flush", 3, 255, 1, 600]):
        if n == "flush":
            p.flush(0)
        else:
            p.append(0, adversarial_tokens(rng, B, H, n), adversarial_tokens(rng, B, H, n))
        p.check_bytes(0)
        if step in (3, 8):
            q = (rng.standard_normal((B, H * G, 128)) / np.sqrt(128)).astype(np.float16)
            got, want = p.decode(0, q, SIGMA)
            assert_attention_close(got, want)
    s = p.ora[0].sched
    assert s.young_head > 0 and any(s.old_demoted)


def test_demotion_saturates_decoded_values():
    """Groups whose maximum is 65504 and whose minimum varies: many decoded young values
    overshoot the fp16 range and are saturated before the old tier quantizes them."""
    rng = np.random.default_rng(5)
    B, H = 1, 2
    p = Pair(1, B, H, 2000, "int4", 128, "int2", 300, demote=True)
    x = rng.uniform(-65504, 65504, size=(B, H, 768, 128))
    for g in (0, 64):
        x[..., g] = 65504
        x[..., g + 1] = -rng.uniform(0, 65504, size=(B, H, 768))
    x = x.astype(np.float16)
    for i in range(6):                       # chunk by chunk: each lands young, then ages
        sl = slice(128 * i, 128 * i + 128)
        p.append(0, x[:, :, sl].copy(), x[:, :, sl, ::-1].copy())
        p.check_bytes(0)
    assert p.ora[0].sched.young_head >= 3 * 128
