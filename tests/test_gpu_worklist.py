"""Launch from a longest-first work list: bitwise the grid launch's results."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceBatch, dev16, dev32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _zipf_lens(seed, B=96):
    rng = np.random.default_rng(seed)
    lens = np.clip(rng.zipf(1.1, size=B), 1, 2048).astype(np.int32)
    lens[5] = 0                                    # an idle slot
    return lens


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
@pytest.mark.parametrize("q8", [False, True], ids=["bf16", "int8"])
@pytest.mark.parametrize("fused", [False, True], ids=["decode", "fused"])
def test_worklist_launch_matches_grid_launch(q8, fused, out_dtype):
    from paged_kv_decode_07_amd import binding as pa
    lens = _zipf_lens(1500 + 2 * q8 + fused)
    pages = int(sum(W.pages_for(L) for L in lens)) + 8
    work_h, ps, ns = pa.decode_worklist(lens, pages, int8=q8, num_cus=256)
    # a bogus entry (sequence outside the batch) must be skipped, not followed
    work_h = np.concatenate([work_h, [[len(lens) + 5, 0], [0, ns + 3]]]).astype(np.int32)
    work = dev32(work_h)
    msl = int(lens.max())
    outs = []
    for use_list in (False, True):
        if q8:
            w = W.make_q8_batch(lens, pages, 1600, append=fused)
            kc, vc, sc = (torch.from_numpy(a.copy()).cuda() for a in (w.k_codes, w.v_codes, w.kv_scales))
            kn = dev16(w.k_new) if fused else None
            vn = dev16(w.v_new) if fused else None
            if use_list:
                out = pa.append_decode_attention_worklist(dev16(w.q), kn, vn, kc, vc, dev32(w.block_tables),
                                                          dev32(w.seq_lens), msl, work, ps, kv_scales=sc,
                                                          out_dtype=out_dtype)
            elif fused:
                out = pa.append_decode_attention_q8(dev16(w.q), kn, vn, kc, vc, sc, dev32(w.block_tables),
                                                    dev32(w.seq_lens), msl, pages_per_split=ps,
                                                    out_dtype=out_dtype)
            else:
                out = pa.decode_attention_q8(dev16(w.q), kc, vc, sc, dev32(w.block_tables),
                                             dev32(w.seq_lens), msl, pages_per_split=ps,
                                             out_dtype=out_dtype)
            pools = (kc, vc, sc.view(torch.int32))
        else:
            w = W.make_batch(lens, pages, 1600, append=fused)
            d = DeviceBatch(w)
            if use_list:
                out = pa.append_decode_attention_worklist(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt,
                                                          d.lens, msl, work, ps, out_dtype=out_dtype)
            elif fused:
                out = pa.append_decode_attention(d.q, d.k_new, d.v_new, d.k_pool, d.v_pool, d.bt, d.lens,
                                                 msl, pages_per_split=ps, out_dtype=out_dtype)
            else:
                out = pa.decode_attention(d.q, d.k_pool, d.v_pool, d.bt, d.lens, msl, pages_per_split=ps,
                                          out_dtype=out_dtype)
            pools = (d.k_pool, d.v_pool)
        torch.cuda.synchronize()
        outs.append((out.clone(), [p.clone() for p in pools]))
    (o0, p0), (o1, p1) = outs
    assert o0.dtype == out_dtype
    assert torch.equal(o0, o1), "work-list launch differs from the grid launch"
    for a, b in zip(p0, p1):
        assert torch.equal(a, b), "pools differ"
    assert torch.all(o0[5] == 0)


def test_ring_depth_leaves_results_bitwise_unchanged():
    """BF16 pages stream through one LDS slot per wavefront or two, chosen per launch from
    the plan (more work-groups than CUs: one slot; at most one per CU with short splits: two).
    The depth changes when pages are requested, not the order they are used in: the grid
    launch of this plan (40 sequences x 8 splits = 320 work-groups: one slot) and its work
    list (40 non-empty 16-page items: two slots) give the same bits, and both match the
    oracle."""
    import oracle
    from gpu_util import assert_close
    from paged_kv_decode_07_amd import binding as pa
    lens = np.random.default_rng(1700).integers(1, 257, size=40).astype(np.int32)
    lens[0], lens[1] = 256, 1                        # a full 16-page split, a one-token one
    w = W.make_batch(lens, int(sum(W.pages_for(L) for L in lens)) + 8, 1701)
    msl, ps = 2048, 16                               # 8 splits per sequence on the grid
    db = DeviceBatch(w)
    work_h, ps_w, _ = pa.decode_worklist(lens, w.num_pages, max_seq_len=msl, pages_per_split=ps,
                                         num_cus=256)
    assert ps_w == ps and len(work_h) == len(lens)   # one item per sequence: 40 <= 256 CUs
    grid = pa.decode_attention(db.q, db.k_pool, db.v_pool, db.bt, db.lens, msl, scale=w.scale,
                               pages_per_split=ps)
    listed = pa.append_decode_attention_worklist(db.q, None, None, db.k_pool, db.v_pool, db.bt,
                                                 db.lens, msl, dev32(work_h), ps, scale=w.scale)
    torch.cuda.synchronize()
    a, b = grid.cpu().numpy(), listed.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = oracle.decode_attention(w.q, w.k_pool, w.v_pool, w.block_tables, w.seq_lens, w.scale)
    assert_close(a.astype(np.float64), ref, where="ring depths")
