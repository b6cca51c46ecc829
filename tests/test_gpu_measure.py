"""The streaming-read calibration reads every word once (its XOR fold proves it)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,groups", [(4, 1), (4096 + 4, 7), (1 << 20, 0), (3 * (1 << 18) + 12, 300)])
def test_stream_read_folds_every_word(words, groups):
    from paged_kv_decode_07_amd import binding as pa
    rng = np.random.default_rng(words + groups)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    pa.stream_read(buf, sink, groups=groups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
