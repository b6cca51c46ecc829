"""Quantised pages (INT8 and INT4): where the pages sit in the pool does not change a
single bit of the result, and the result repeats bit for bit from run to run.

The same logical cache is laid out once through a seeded random permutation of the pool
and once in pool order; the block tables differ, the outputs must not.  Split sizes of
3 and 16 pages run one wavefront per KV head; 128-page splits of this small batch run
two on INT4 pages (each takes half of a split and the two states merge in LDS).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev16, dev32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _decode(w, nbits, ps):
    from paged_kv_decode_07_amd import binding as pa
    kc, vc, sc = (torch.from_numpy(np.ascontiguousarray(a)).cuda()
                  for a in (w.k_codes, w.v_codes, w.kv_scales))
    fn = pa.decode_attention_q8 if nbits == 8 else pa.decode_attention_q4
    out = fn(dev16(w.q), kc, vc, sc, dev32(w.block_tables), dev32(w.seq_lens), w.max_seq_len,
             scale=w.scale, pages_per_split=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("ps", [3, 16, 128])
@pytest.mark.parametrize("nbits", [8, 4], ids=["int8", "int4"])
def test_quant_decode_page_shuffle_bitwise_and_repeatable(nbits, ps):
    lens = [3, 40, 129, 700, 2048]
    pages = sum(W.pages_for(L) for L in lens) + 7
    shuffled = W.make_q8_batch(lens, pages, 4300 + nbits, nbits=nbits)
    ordered = W.make_q8_batch(lens, pages, 4300 + nbits, placement="identity", nbits=nbits)
    assert not np.array_equal(shuffled.block_tables, ordered.block_tables)
    got = _decode(shuffled, nbits, ps)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, _decode(ordered, nbits, ps)), "depends on page placement"
    for _ in range(2):
        assert np.array_equal(_decode(shuffled, nbits, ps), got), "not repeatable"
