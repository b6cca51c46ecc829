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
