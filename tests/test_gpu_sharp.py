"""Sharp scores on the GPU: the online softmax's rescale, on every page format.

The FP32 online softmax keeps a running maximum and rescales what it has
summed when a later score passes it (the samir-vllm README's paged decode
attention, "features completed so far"; the max subtraction of the
coreui.cn article, section 3.2).  With N(0, 1) inputs at scale 1/8 the
maximum is essentially never raised after the first page, so these tests use
the sharp generator (``workloads.make_sharp_batch``): ramps of key magnitude
up and down, a query-aligned spike on the last token (in a part-filled last
page; appended by the fused step), a spike mid-sequence, and scale 2.0.
A CPU test of the generator pins that these inputs do raise a page-wise
running maximum far past its first value.

Every case runs the two-call form (append, then decode) and the fused step
with splits of 1, 3, 16 and 128 pages and the library's own plan, so the
split merge sees maxima far apart; pools are compared bit for bit and every
output element against the float64 oracle (max-abs 2e-3, relative 1e-2).
INT8 and INT4 pages are quantised on the GPU from the same BF16 rows
(``pa_fill_kv_q8`` / ``_q4``); their codes and scales must equal the
oracle's quantiser's, and the attention is compared with the oracle over the
oracle's own pools.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DeviceBatch, assert_close, dev16, dev32, gpu_append, gpu_decode, gpu_fused, host16
from oracle import kvquant

pytestmark = pytest.mark.gpu

LENS = [37, 100, 255, 256, 1000, 2047, 2048, 17, 1, 0]
SPLITS = [0, 1, 3, 16, 128]
SEED = {m: 7100 + i for i, m in enumerate(W.SHARP_MODES)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _pa():
    from paged_kv_decode_07_amd import binding as pa
    return pa


def _batch(mode):
    return W.make_sharp_batch(LENS, sum(W.pages_for(L) for L in LENS) + 11, SEED[mode], mode,
                              append=True)


# ---------------------------------------------------------------------------
# BF16 pages
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pages_per_split", SPLITS)
@pytest.mark.parametrize("mode", W.SHARP_MODES)
def test_sharp_bf16_two_call_and_fused(mode, pages_per_split):
    print(f"sharp bf16 {mode} ps={pages_per_split}", flush=True)
    w = _batch(mode)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    a = DeviceBatch(w)
    gpu_append(a)
    assert np.array_equal(host16(a.k_pool), k_ref) and np.array_equal(host16(a.v_pool), v_ref)
    two = gpu_decode(a, pages_per_split=pages_per_split)
    assert_close(two, ref, where=f"bf16 {mode} two-call ps={pages_per_split}")
    f = DeviceBatch(w)
    fused = gpu_fused(f, pages_per_split=pages_per_split)
    assert np.array_equal(host16(f.k_pool), k_ref) and np.array_equal(host16(f.v_pool), v_ref)
    assert_close(fused, ref, where=f"bf16 {mode} fused ps={pages_per_split}")
    assert np.array_equal(fused, two), "fused output differs from append + decode"
    assert np.all(fused[-1] == 0.0)


@pytest.mark.parametrize("mode", ["ramp_up", "tail_max", "scale2"])
def test_sharp_bf16_output(mode):
    w = _batch(mode)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    got = gpu_fused(DeviceBatch(w), pages_per_split=3, out_dtype=torch.bfloat16)
    assert_close(got, ref, bf16_out=True, where=f"bf16 out {mode}")


@pytest.mark.parametrize("mode", ["ramp_up", "tail_max", "scale2"])
def test_sharp_bf16_work_list(mode):
    pa = _pa()
    w = _batch(mode)
    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                    w.seq_lens)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    for ps in (1, 16):
        wl, wps, _ = pa.decode_worklist(w.seq_lens, w.num_pages, pages_per_split=ps)
        d = DeviceBatch(w)
        out = pa.append_decode_attention_worklist(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt,
                                                  d.lens, w.max_seq_len, dev32(wl), wps,
                                                  scale=w.scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), ref, where=f"work list {mode} ps={ps}")


# ---------------------------------------------------------------------------
# INT8 and INT4 pages, quantised on the GPU from the same BF16 rows
# ---------------------------------------------------------------------------
def _empty_pools(npg, nbits):
    width, dt = (64, np.int8) if nbits == 8 else (32, np.uint8)
    return (np.zeros((npg, 8, 16, width), dt), np.zeros((npg, 8, 16, width), dt),
            np.full((npg, 8, 2, 16), np.nan, np.float32))


def _quantised(w, nbits):
    """(device pools filled by the GPU, the oracle's pools) for the stored tokens."""
    pa = _pa()
    kc, vc, sc = _empty_pools(w.num_pages, nbits)
    dk, dv, ds = (torch.from_numpy(x.copy()).cuda() for x in (kc, vc, sc))
    for b, L in enumerate(w.seq_lens):
        stored = int(L) - 1                           # the last token comes with the append
        if stored <= 0:
            continue
        kr = W.logical_rows(w.k_pool, w.block_tables[b], stored)
        vr = W.logical_rows(w.v_pool, w.block_tables[b], stored)
        pa.fill_kv_q8(dev16(kr), dev16(vr), dev32(w.block_tables[b]), 0, dk, dv, ds, nbits=nbits)
        kc, vc, sc = kvquant.fill_kv_q8(kc, vc, sc, kr, vr, w.block_tables[b], 0, nbits=nbits)
    torch.cuda.synchronize()
    return (dk, dv, ds), (kc, vc, sc)


def _same(dev_pools, pools, what):
    dk, dv, ds = (t.cpu().numpy() for t in dev_pools)
    assert np.array_equal(dk, pools[0]), f"{what}: K codes"
    assert np.array_equal(dv, pools[1]), f"{what}: V codes"
    assert np.array_equal(ds.view(np.uint32), pools[2].view(np.uint32)), f"{what}: scales"


@pytest.mark.parametrize("nbits", [8, 4])
@pytest.mark.parametrize("pages_per_split", SPLITS)
@pytest.mark.parametrize("mode", W.SHARP_MODES)
def test_sharp_quantised_two_call_and_fused(mode, pages_per_split, nbits):
    print(f"sharp int{nbits} {mode} ps={pages_per_split}", flush=True)
    pa = _pa()
    w = _batch(mode)
    dev_pools, pools = _quantised(w, nbits)
    _same(dev_pools, pools, "fill")
    post = kvquant.append_kv_q8(*pools, w.k_new, w.v_new, w.block_tables, w.seq_lens,
                                nbits=nbits)
    ref = kvquant.decode_attention_q8(w.q, *post, w.block_tables, w.seq_lens, w.scale,
                                      nbits=nbits)
    q, kn, vn = dev16(w.q), dev16(w.k_new), dev16(w.v_new)
    bt, lens = dev32(w.block_tables), dev32(w.seq_lens)
    # two calls: quantised append, then decode
    a = tuple(t.clone() for t in dev_pools)
    pa.append_kv_q8(kn, vn, *a, bt, lens, nbits=nbits)
    two = pa.decode_attention_q8(q, *a, bt, lens, w.max_seq_len, scale=w.scale,
                                 pages_per_split=pages_per_split, nbits=nbits)
    torch.cuda.synchronize()
    _same(a, post, "append")
    two = two.cpu().numpy().astype(np.float64)
    assert_close(two, ref, where=f"int{nbits} {mode} two-call ps={pages_per_split}")
    # the fused step
    f = tuple(t.clone() for t in dev_pools)
    fused = pa.append_decode_attention_q8(q, kn, vn, *f, bt, lens, w.max_seq_len, scale=w.scale,
                                          pages_per_split=pages_per_split, nbits=nbits)
    torch.cuda.synchronize()
    _same(f, post, "fused append")
    fused = fused.cpu().numpy().astype(np.float64)
    assert_close(fused, ref, where=f"int{nbits} {mode} fused ps={pages_per_split}")
    assert np.array_equal(fused, two), "fused output differs from append + decode"


@pytest.mark.parametrize("nbits", [8, 4])
def test_sharp_quantised_work_list(nbits):
    pa = _pa()
    w = _batch("ramp_up")
    dev_pools, pools = _quantised(w, nbits)
    post = kvquant.append_kv_q8(*pools, w.k_new, w.v_new, w.block_tables, w.seq_lens,
                                nbits=nbits)
    ref = kvquant.decode_attention_q8(w.q, *post, w.block_tables, w.seq_lens, w.scale,
                                      nbits=nbits)
    for ps in (1, 16, 128):
        wl, wps, _ = pa.decode_worklist(w.seq_lens, w.num_pages, pages_per_split=ps,
                                        int8=nbits == 8, int4=nbits == 4)
        d = tuple(t.clone() for t in dev_pools)
        out = pa.append_decode_attention_worklist(
            dev16(w.q), dev16(w.k_new), dev16(w.v_new), d[0], d[1], dev32(w.block_tables),
            dev32(w.seq_lens), w.max_seq_len, dev32(wl), wps, scale=w.scale, kv_scales=d[2])
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), ref,
                     where=f"int{nbits} work list ps={ps}")
