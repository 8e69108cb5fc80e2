"""GPU: the read probe (measurement aid) reads every 32-bit word of its buffer exactly once:
the XOR of the sink equals the XOR of the buffer, for a size that is not a multiple of the
launch's grid stride and for a single 16-byte row."""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, (64 << 20) + 48])
def test_read_probe_reads_every_word_once(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).to("cuda")
    sink = torch.full((kvq.read_probe_sink_bytes(),), 0x5A, dtype=torch.uint8, device="cuda")
    kvq.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
