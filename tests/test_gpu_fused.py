"""Fused append + decode (one launch) against the two-call sequence and the oracle.

The fused call must leave the pools bit-identical to pa_append_kv and return
outputs bit-identical to pa_decode_attention run after it (same arithmetic,
the new token taken from registers instead of the pool), and within the
attention tolerance of the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DeviceBatch, assert_close, gpu_append, gpu_decode, gpu_fused, host16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _two_call_vs_fused(batch, ps):
    a = DeviceBatch(batch)
    gpu_append(a)
    two = gpu_decode(a, pages_per_split=ps)
    f = DeviceBatch(batch)
    fused = gpu_fused(f, pages_per_split=ps)
    assert np.array_equal(host16(f.k_pool), host16(a.k_pool)), "K pool differs"
    assert np.array_equal(host16(f.v_pool), host16(a.v_pool)), "V pool differs"
    assert np.array_equal(fused, two), "fused output differs from append + decode"
    return fused


@pytest.mark.parametrize("pages_per_split", [0, 1, 3, 16, 128])
def test_fused_edge_lengths(pages_per_split):
    lens = [1, 2, 15, 16, 17, 32, 33, 100, 2047, 2048, 0]
    w = W.make_batch(lens, sum(W.pages_for(L) for L in lens) + 9, seed=71, append=True)
    got = _two_call_vs_fused(w, pages_per_split)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(got, ref, where=f"fused edge ps={pages_per_split}")
    assert np.all(got[-1] == 0.0)


def test_fused_seq_len_one_returns_the_new_v_row():
    w = W.make_batch([1] * 5, 8, seed=72, append=True)
    got = gpu_fused(DeviceBatch(w))
    for b in range(5):
        vnew = oracle.bf16_bits_to_f64(w.v_new[b])
        for h in range(32):
            assert np.array_equal(got[b, h], vnew[h // 4])


@pytest.mark.parametrize("wi", [5, 6], ids=["zipf-clipped", "zipf-truncated"])
def test_fused_full_batch512_zipf(wi):
    w = W.make_workload(wi)
    got = _two_call_vs_fused(w, 0)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(got, ref, where=f"fused batch512 (workload {wi}) every sequence")


def test_fused_full_batch256_len2048_bench_configuration():
    w = W.make_workload(4, append=True)
    got = _two_call_vs_fused(w, 0)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(got, ref, where="fused batch256 every sequence")


def test_fused_16_layer_workload_every_layer():
    for layer in range(W.NUM_LAYERS_W3):
        print(f"fused: 16-layer workload, layer {layer}", flush=True)
        w = W.make_workload(3, layer=layer)
        got = _two_call_vs_fused(w, 0)
        k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                        w.seq_lens)
        ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
        assert_close(got, ref, where=f"fused 16-layer layer {layer}")


def test_fused_bad_last_page_writes_nothing_and_gives_nan():
    w = W.make_batch([20, 40, 5], 16, seed=73, append=True)
    bt = w.block_tables.copy()
    bt[1, (40 - 1) // 16] = 999                       # the page the append would write
    db = DeviceBatch(w)
    from gpu_util import dev32
    db.bt = dev32(bt)
    got = gpu_fused(db)
    assert np.all(np.isnan(got[1]))
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new[[0, 2]], w.v_new[[0, 2]],
                                    bt[[0, 2]], w.seq_lens[[0, 2]])
    assert np.array_equal(host16(db.k_pool), k_ref)
    assert np.array_equal(host16(db.v_pool), v_ref)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(got[[0, 2]], ref[[0, 2]], where="fused others")


def test_fused_batch_of_70000_single_token_sequences():
    """A batch larger than 65,535 (one block per sequence in a one-dimensional
    grid): every sequence holds only its appended token, so each output row is
    that token's V row exactly (softmax over one token)."""
    from paged_kv_decode_07_amd import binding as pa
    B = 70000
    gen = torch.Generator(device="cuda").manual_seed(70000)
    rows = lambda: torch.randn((B, 8, 64), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, 32, 64), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    kn, vn = rows(), rows()
    k_pool = torch.zeros((B, 16, 8, 64), dtype=torch.int16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    bt = torch.full((B, W.MAX_BLOCKS), -1, dtype=torch.int32, device="cuda")
    bt[:, 0] = torch.randperm(B, generator=gen, device="cuda").to(torch.int32)
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    print(f"fused batch {B}, seq_len 1", flush=True)
    out = pa.append_decode_attention(q, kn.view(torch.int16), vn.view(torch.int16), k_pool, v_pool,
                                     bt, lens, 1)
    torch.cuda.synchronize()
    want = vn.float().repeat_interleave(4, dim=1)                # head h reads KV head h // 4
    assert torch.equal(out, want)
    page = bt[:, 0].long()
    assert torch.equal(v_pool[page, 0], vn.view(torch.int16))
    assert torch.equal(k_pool[page, 0], kn.view(torch.int16))


OVER = [40, 300, 17, 129]          # with max_seq_len 100, sequences 1 and 3 are over it


@pytest.mark.parametrize("pages_per_split", [0, 3])
def test_fused_over_length_appends_like_the_two_call_form(pages_per_split):
    """A length above max_seq_len (but within the block table) gets a NaN
    output row from both forms, and its new row is written by both, as the
    separate append writes every row within the table's capacity."""
    from gpu_util import dev16
    from paged_kv_decode_07_amd import binding as pa
    w = W.make_batch(OVER, sum(W.pages_for(L) for L in OVER) + 5, seed=74, append=True)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    a = DeviceBatch(w)
    gpu_append(a)
    two = pa.decode_attention(a.q, a.k_pool, a.v_pool, a.bt, a.lens, 100,
                              pages_per_split=pages_per_split)
    f = DeviceBatch(w)
    fused = pa.append_decode_attention(f.q, f.k_new, f.v_new, f.k_pool, f.v_pool, f.bt, f.lens,
                                       100, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    for d in (a, f):
        assert np.array_equal(host16(d.k_pool), k_ref) and np.array_equal(host16(d.v_pool), v_ref)
    two, fused = two.cpu().numpy(), fused.cpu().numpy()
    for b in (1, 3):
        assert np.all(np.isnan(two[b])) and np.all(np.isnan(fused[b]))
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    assert_close(fused[[0, 2]].astype(np.float64), ref[[0, 2]], where="over-length others")
    assert np.array_equal(fused[[0, 2]], two[[0, 2]])
    # with RoPE: tables covering the capacity, both forms rotate and write every row
    cos, sin = W.rope_table()
    rc, rs = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    a = DeviceBatch(w)
    pa.append_kv_rope(a.q, a.k_new, a.v_new, rc, rs, a.k_pool, a.v_pool, a.bt, a.lens)
    f = DeviceBatch(w)
    pa.append_decode_attention_rope(f.q, f.k_new, f.v_new, rc, rs, f.k_pool, f.v_pool, f.bt,
                                    f.lens, 100, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    _, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    k_rref, v_rref = oracle.append_kv(w.k_pool, w.v_pool, k_rot, w.v_new, w.block_tables,
                                      w.seq_lens)
    for d in (a, f):
        assert np.array_equal(host16(d.k_pool), k_rref)
        assert np.array_equal(host16(d.v_pool), v_rref)


@pytest.mark.parametrize("nbits", [8, 4])
def test_fused_quantised_over_length_appends_like_the_two_call_form(nbits):
    from gpu_util import dev16, dev32
    from oracle import kvquant
    from paged_kv_decode_07_amd import binding as pa
    w = W.make_q8_batch(OVER, sum(W.pages_for(L) for L in OVER) + 5, 75, append=True,
                        nbits=nbits)
    want = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                w.block_tables, w.seq_lens, nbits=nbits)
    q, kn, vn = dev16(w.q), dev16(w.k_new), dev16(w.v_new)
    bt, lens = dev32(w.block_tables), dev32(w.seq_lens)

    def pools():
        return tuple(torch.from_numpy(np.ascontiguousarray(x)).cuda()
                     for x in (w.k_codes, w.v_codes, w.kv_scales))
    a = pools()
    pa.append_kv_q8(kn, vn, *a, bt, lens, nbits=nbits)
    two = pa.decode_attention_q8(q, *a, bt, lens, 100, nbits=nbits)
    f = pools()
    fused = pa.append_decode_attention_q8(q, kn, vn, *f, bt, lens, 100, nbits=nbits)
    torch.cuda.synchronize()
    for d in (a, f):
        got = [t.cpu().numpy() for t in d]
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    two, fused = two.cpu().numpy(), fused.cpu().numpy()
    for b in (1, 3):
        assert np.all(np.isnan(two[b])) and np.all(np.isnan(fused[b]))
    assert np.array_equal(fused[[0, 2]], two[[0, 2]])
