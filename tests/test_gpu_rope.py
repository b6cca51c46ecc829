"""RoPE fused with the append (row NEXT-2) on the GPU against the oracle.

The rotated key written to the pool and the rotated query are compared bit
for bit with the oracle (both round the float32 rotation to BF16 to nearest
even); the fused RoPE decode step must equal the two-call form bitwise and
the oracle's attention on the rotated cache within the attention bound.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DeviceBatch, assert_close, dev32, host16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _tables(positions=W.MAX_CONTEXT):
    cos, sin = W.rope_table(positions)
    return cos, sin, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()


def _oracle_step(w, cos, sin):
    q_rot, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, k_rot, w.v_new, w.block_tables,
                                    w.seq_lens)
    return q_rot, k_ref, v_ref


def test_append_rope_bitexact_edge_lengths():
    from paged_kv_decode_07_amd import binding as pa
    cos, sin, cos_d, sin_d = _tables()
    lens = [1, 2, 15, 16, 17, 33, 1000, 2047, 2048, 0]
    w = W.make_batch(lens, sum(W.pages_for(L) for L in lens) + 5, seed=81, append=True)
    db = DeviceBatch(w)
    q_out = pa.append_kv_rope(db.q, db.k_new, db.v_new, cos_d, sin_d, db.k_pool, db.v_pool,
                              db.bt, db.lens)
    torch.cuda.synchronize()
    q_rot, k_ref, v_ref = _oracle_step(w, cos, sin)
    assert np.array_equal(host16(q_out), q_rot)
    assert np.array_equal(host16(db.k_pool), k_ref)
    assert np.array_equal(host16(db.v_pool), v_ref)


def test_append_rope_bitexact_full_batch512():
    from paged_kv_decode_07_amd import binding as pa
    cos, sin, cos_d, sin_d = _tables()
    w = W.make_workload(5)
    db = DeviceBatch(w)
    q_out = pa.append_kv_rope(db.q, db.k_new, db.v_new, cos_d, sin_d, db.k_pool, db.v_pool,
                              db.bt, db.lens)
    torch.cuda.synchronize()
    q_rot, k_ref, v_ref = _oracle_step(w, cos, sin)
    assert np.array_equal(host16(q_out), q_rot)
    assert np.array_equal(host16(db.k_pool), k_ref)
    assert np.array_equal(host16(db.v_pool), v_ref)


@pytest.mark.parametrize("pages_per_split", [0, 2, 16])
def test_fused_rope_equals_two_calls_and_oracle(pages_per_split):
    from paged_kv_decode_07_amd import binding as pa
    cos, sin, cos_d, sin_d = _tables()
    lens = [1, 3, 16, 17, 300, 2048, 0]
    w = W.make_batch(lens, sum(W.pages_for(L) for L in lens) + 5, seed=82, append=True)
    a = DeviceBatch(w)
    q_out = pa.append_kv_rope(a.q, a.k_new, a.v_new, cos_d, sin_d, a.k_pool, a.v_pool, a.bt,
                              a.lens)
    two = pa.decode_attention(q_out, a.k_pool, a.v_pool, a.bt, a.lens, w.max_seq_len,
                              pages_per_split=pages_per_split)
    f = DeviceBatch(w)
    fused = pa.append_decode_attention_rope(f.q, f.k_new, f.v_new, cos_d, sin_d, f.k_pool,
                                            f.v_pool, f.bt, f.lens, w.max_seq_len,
                                            pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    assert np.array_equal(host16(f.k_pool), host16(a.k_pool))
    assert np.array_equal(fused.cpu().numpy(), two.cpu().numpy())
    q_rot, k_ref, v_ref = _oracle_step(w, cos, sin)
    ref = oracle.decode_attention(q_rot, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(fused.cpu().numpy().astype(np.float64), ref, where=f"rope ps={pages_per_split}")


def test_rope_rejects_short_tables():
    from paged_kv_decode_07_amd import binding as pa
    cos, sin, cos_d, sin_d = _tables(100)
    w = W.make_batch([50, 60], 16, seed=83, append=True)
    db = DeviceBatch(w)
    with pytest.raises(RuntimeError, match="VALUE"):
        pa.append_kv_rope(db.q, db.k_new, db.v_new, cos_d, sin_d, db.k_pool, db.v_pool,
                          db.bt, db.lens)            # capacity 2048 > 100 positions
    out = pa.append_decode_attention_rope(db.q, db.k_new, db.v_new, cos_d, sin_d, db.k_pool,
                                          db.v_pool, db.bt, db.lens, 60)     # 60 <= 100: fine
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out.cpu().numpy()))
