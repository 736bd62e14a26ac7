"""The streaming-read probe reads every 32-bit word exactly once (its XOR checksums match)."""

import numpy as np
import pytest
import torch

from paged_kv_cache_220_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 32768 * 3 + 48, 64 << 20, (32768 << 12) + 32768 + 16])
def test_read_probe_checksum(nbytes):
    rng = np.random.default_rng([220, 77, nbytes % 1000003])
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    want = np.bitwise_xor.reduce(host)
    dev = torch.device("cuda:0")
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.full((B.PROBE_SINK_WORDS,), -1, dtype=torch.int32, device=dev)
    n = B.pa_read_probe(buf, sink)
    torch.cuda.synchronize()
    words = sink.cpu().numpy().view(np.uint32)
    assert n == min(-(-nbytes // B.PROBE_CHUNK_BYTES), B.PROBE_SINK_WORDS)
    assert np.bitwise_xor.reduce(words[:n]) == want
    assert np.all(words[n:] == 0xFFFFFFFF)          # words past the launch untouched
