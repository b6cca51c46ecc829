"""Prefill page fill (row NEXT-3) and a decode loop driven by the page allocator.

The fill is compared bit for bit with the oracle.  The loop runs a few
requests through the C++ allocator (admission, lazy pages, early finish,
re-admission into the freed credit); its block tables drive the prompt fill
and the fused append + decode of every layer and step on the GPU, and the
oracle recomputes every step's attention from its own copy of the cache.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close, dev16, dev32, host16

pytestmark = pytest.mark.gpu

HKV, D, P = W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("start,count", [(0, 1), (0, 37), (5, 16), (16, 17), (0, 2048), (1000, 1048)])
def test_fill_bitexact(start, count):
    from paged_kv_decode_07_amd import binding as pa
    rng = np.random.default_rng(start * 7 + count)
    pages = 200
    k_pool = np.full((pages, P, HKV, D), W.BF16_NAN, np.uint16)
    v_pool = k_pool.copy()
    row = np.full(128, -1, np.int32)
    n = W.pages_for(start + count)
    row[:n] = rng.permutation(pages)[:n]
    kr = W.random_rows(rng, count)
    vr = W.random_rows(rng, count)
    kd, vd = dev16(k_pool), dev16(v_pool)
    pa.fill_kv(dev16(kr), dev16(vr), dev32(row), start, kd, vd)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.fill_kv(k_pool, v_pool, kr, vr, row, start)
    assert np.array_equal(host16(kd), k_ref) and np.array_equal(host16(vd), v_ref)


@pytest.mark.parametrize("launch", ["grid", "worklist", "balanced1", "balanced8"])
def test_allocator_driven_decode_loop(launch):
    """Every step re-plans its launch from the current lengths (the work list and
    the balanced plan are host plans for one batch of lengths), as a serving
    loop does."""
    from paged_kv_decode_07_amd import binding as pa
    layers, pool_pages, steps = 2, 40, 40      # credit 10+8+18 fits, 6 and 16 must wait
    rng = np.random.default_rng(501)
    alloc = pa.KVPool(pool_pages, layers, P, W.MAX_CONTEXT)
    # requests: (prompt tokens, new tokens allowed); credit = layers * ceil((p + n - 1) / 16)
    reqs = {0: (30, 40), 1: (5, 60), 2: (100, 30), 3: (17, 20), 4: (64, 50)}
    for rid, (p, n) in reqs.items():
        assert alloc.submit(rid, p, n) == "wait"
    k_pool = np.full((pool_pages, P, HKV, D), W.BF16_NAN, np.uint16)
    v_pool = k_pool.copy()
    kd, vd = dev16(k_pool), dev16(v_pool)
    length, finish_at = {}, {0: 25, 1: 999, 2: 12, 3: 999, 4: 999}
    checked = 0
    for step in range(steps):
        for rid in alloc.admit():                       # prefill the newly admitted
            p = reqs[rid][0]
            alloc.grow(rid, p)
            for layer in range(layers):
                row = np.full(128, -1, np.int32)
                bt = alloc.block_table(rid, layer)
                row[:len(bt)] = bt
                kr, vr = W.random_rows(rng, p), W.random_rows(rng, p)
                pa.fill_kv(dev16(kr), dev16(vr), dev32(row), 0, kd, vd)
                k_pool, v_pool = oracle.fill_kv(k_pool, v_pool, kr, vr, row, 0)
            length[rid] = p
        active = sorted(length)
        if not active:
            break
        for rid in active:                              # one new token each
            length[rid] += 1
            alloc.grow(rid, length[rid])
        alloc.step()
        B = len(active)
        lens = np.array([length[r] for r in active], np.int32)
        q = W.random_q(rng, B)
        for layer in range(layers):
            bts = np.full((B, 128), -1, np.int32)
            for i, rid in enumerate(active):
                bt = alloc.block_table(rid, layer)
                bts[i, :len(bt)] = bt
            kn, vn = W.random_rows(rng, B), W.random_rows(rng, B)
            msl = int(lens.max())
            if launch == "grid":
                out = pa.append_decode_attention(dev16(q), dev16(kn), dev16(vn), kd, vd,
                                                 dev32(bts), dev32(lens), msl, scale=W.SCALE)
            elif launch == "worklist":
                work, ps, _ = pa.decode_worklist(lens, pool_pages, max_seq_len=msl)
                out = pa.append_decode_attention_worklist(
                    dev16(q), dev16(kn), dev16(vn), kd, vd, dev32(bts), dev32(lens), msl,
                    torch.from_numpy(work).cuda(), ps, scale=W.SCALE)
            else:
                plan = pa.balance_plan(lens, pool_pages, max_seq_len=msl,
                                       heads_together=int(launch[-1]))
                out = pa.decode_balanced(dev16(q), kd, vd, dev32(bts), dev32(lens), msl, plan,
                                         k_new=dev16(kn), v_new=dev16(vn), scale=W.SCALE)
            k_pool, v_pool = oracle.append_kv(k_pool, v_pool, kn, vn, bts, lens)
            ref = oracle.decode_attention(q, k_pool, v_pool, bts, lens, W.SCALE)
            assert_close(out.cpu().numpy().astype(np.float64), ref,
                         where=f"{launch} step {step} layer {layer}")
            checked += 1
        for rid in active:                              # finish: budget used up or early stop
            p, n = reqs[rid]
            if length[rid] >= p + n - 1 or step == finish_at[rid]:
                alloc.finish(rid)
                del length[rid]
    torch.cuda.synchronize()
    assert np.array_equal(host16(kd), k_pool) and np.array_equal(host16(vd), v_pool)
    st = alloc.stats
    assert checked >= 40 and st["admission_waits"] >= 1 and st["peak_active"] >= 3
