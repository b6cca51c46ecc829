"""The allocation-free fused step against the fused step with a caller workspace.

pa_append_decode_attention_noalloc keeps the split partials in the library's
own device scratch.  Two calls in a row, the second with a smaller batch and
shorter splits (so it reads scratch rows that the first call left behind
unless it writes them first), must each give the outputs and pools of
pa_append_decode_attention on the same inputs bit for bit, and match the
oracle within the attention tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DeviceBatch, assert_close, host16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


CALLS = [
    # (lengths, pages per split, output dtype)
    ([37, 2048, 700, 1, 129, 1500, 16, 900, 2047, 333], 4, torch.float32),
    ([300, 50, 17], 2, torch.bfloat16),
]


def _one(lens, ps, out_dtype, seed):
    from paged_kv_decode_07_amd import binding as pa
    w = W.make_batch(lens, sum(W.pages_for(L) for L in lens) + 7, seed=seed, append=True)
    print(f"no-alloc: batch {len(lens)}, pages per split {ps}, {out_dtype}", flush=True)
    need = pa.decode_workspace_bytes(w.batch, w.max_seq_len, w.num_pages, 128, ps)
    assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES           # the scratch is used
    a = DeviceBatch(w)
    ref_out = pa.append_decode_attention(a.q, a.k_new, a.v_new, a.k_pool, a.v_pool, a.bt, a.lens,
                                         w.max_seq_len, scale=w.scale, out_dtype=out_dtype,
                                         pages_per_split=ps)
    f = DeviceBatch(w)
    out = torch.full((w.batch, 32, 64), float("nan"), dtype=out_dtype, device="cuda")
    got = pa.append_decode_attention_noalloc(f.q, f.k_new, f.v_new, f.k_pool, f.v_pool, f.bt,
                                             f.lens, w.max_seq_len, out, scale=w.scale,
                                             out_dtype=out_dtype, pages_per_split=ps)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(out.view(torch.int16) if out_dtype == torch.bfloat16 else out.view(torch.int32),
                       ref_out.view(torch.int16) if out_dtype == torch.bfloat16
                       else ref_out.view(torch.int32)), "differs from the workspace form"
    assert np.array_equal(host16(f.k_pool), host16(a.k_pool))
    assert np.array_equal(host16(f.v_pool), host16(a.v_pool))
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    assert np.array_equal(host16(f.k_pool), k_ref) and np.array_equal(host16(f.v_pool), v_ref)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(out.float().cpu().numpy().astype(np.float64), ref,
                 bf16_out=out_dtype == torch.bfloat16, where=f"no-alloc batch {len(lens)}")


def test_noalloc_two_calls_in_a_row_match_the_workspace_form():
    for i, (lens, ps, dt) in enumerate(CALLS):
        _one(lens, ps, dt, seed=6100 + i)


def test_noalloc_refuses_partials_beyond_its_scratch():
    from paged_kv_decode_07_amd import binding as pa
    B = 8192
    need = pa.decode_workspace_bytes(B, 2048, 16, 128, 8)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 32, 64), dtype=torch.int16, device="cuda")
    rows = torch.zeros((B, 8, 64), dtype=torch.int16, device="cuda")
    pool = torch.zeros((16, 16, 8, 64), dtype=torch.int16, device="cuda")
    bt = torch.full((B, 128), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, 32, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        pa.append_decode_attention_noalloc(q, rows, rows, pool, pool.clone(), bt, lens, 2048,
                                           out, pages_per_split=8)
