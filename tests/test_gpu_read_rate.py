"""csa2_read_rate (the achievable-read-rate probe): every 16-byte word of the
buffer is read exactly once, so the XOR of all sink words equals the XOR of
all 32-bit words of the buffer, for sizes with and without a partial round."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from fp4_kv_cache_e4m3_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 1001, 65536, (64 << 20) // 16 + 3])
def test_read_rate_reads_every_word_once(n16):
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 1 << 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.zeros(B.READ_RATE_SINK_WORDS, dtype=torch.int32, device="cuda")
    csa2.read_rate(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
