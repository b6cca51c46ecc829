"""Pages beyond the first 4 GiB of a pool: page offsets are formed in 64 bits.

A small batch (lengths 1, 17, 300, 2048 and 33, one new token each) is drawn
by the seeded generators into a small pool.  Its pages are then copied to
pages whose byte offsets all lie past 2^32 in a device pool of a little over
4 GiB per K or V (code) pool, and every other page of that pool stays poisoned.
On it, for BF16, INT8 and INT4 pages:

* the fused append + decode writes each new row into its high page exactly as
  the oracle's append does (every placed page compared), leaves every other
  page of the pool poisoned, and attends within the tolerance of the oracle
  over the small pools;
* decode over the appended pools through a multi-split grid (with the merge),
  the work list and the balanced launch matches the oracle as well.

The block table is the small batch's with every page id mapped to its high
page ("6 Hours of YouTube ...", samir-vllm README, features completed so far:
a page map per sequence into one shared pool).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close, dev16, dev32, host16
from oracle import kvquant

pytestmark = pytest.mark.gpu

LENS = [1, 17, 300, 2048, 33]
EXTRA = 4096                 # pool pages beyond the 4 GiB offset


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pa():
    from paged_kv_decode_07_amd import binding as pa
    return pa


def _say(msg):
    print(msg, flush=True)


def _high_map(small_pages: int, page_bytes: int, seed: int):
    """Pool size and, for each small page id, a distinct page whose byte offset is >= 2^32."""
    first = (1 << 32) // page_bytes
    total = first + EXTRA
    rng = np.random.default_rng(seed)
    hi = (first + rng.permutation(EXTRA)[:small_pages]).astype(np.int64)
    return total, hi


def _map_table(table: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return np.where(table >= 0, hi[np.maximum(table, 0)], -1).astype(np.int32)


def _touched_pages(pool: torch.Tensor, poison: torch.Tensor) -> np.ndarray:
    """Ids of the pages holding anything but the poison value (compared bitwise)."""
    flat = pool.view(pool.shape[0], -1)
    return torch.nonzero((flat != poison).any(dim=1)).flatten().cpu().numpy()


def _check_launches(decode, q_ref_out, lens, total, msl, where, int8=False, int4=False):
    """Decode-only launches over the appended pools against the oracle output."""
    pa = _pa()
    lens_h = np.asarray(lens, np.int32)
    got = decode("grid", dict(pages_per_split=3))
    assert_close(got, q_ref_out, where=f"{where} grid ps=3")
    work, ps, _ = pa.decode_worklist(lens_h, total, 128, msl, pages_per_split=8, int8=int8,
                                     int4=int4)
    got = decode("worklist", dict(work=torch.from_numpy(work).cuda(), pages_per_split=ps))
    assert_close(got, q_ref_out, where=f"{where} work list")
    for h in (8, 1):
        plan = pa.balance_plan(lens_h, total, 128, msl, heads_together=h)
        got = decode("balanced", dict(plan=plan))
        assert_close(got, q_ref_out, where=f"{where} balanced h={h}")


def test_bf16_pages_past_4_gib():
    pa = _pa()
    small_pages = sum(W.pages_for(L) for L in LENS) + 7
    w = W.make_batch(LENS, small_pages, 4401, append=True)
    total, hi = _high_map(small_pages, W.PAGE_SIZE * W.NUM_KV_HEADS * W.HEAD_DIM * 2, 4402)
    _say(f"bf16: pool of {total} pages ({total * 16384 / 2**30:.2f} GiB per pool), pages "
         f"{hi.min()} .. {hi.max()}")
    poison = torch.tensor(np.array([W.BF16_NAN], np.uint16).view(np.int16)[0], device="cuda")
    hi_t = torch.from_numpy(hi).cuda()
    kp = torch.full((total, 16, 8, 64), int(poison), dtype=torch.int16, device="cuda")
    vp = torch.full_like(kp, int(poison))
    kp[hi_t] = dev16(w.k_pool)
    vp[hi_t] = dev16(w.v_pool)
    bt = dev32(_map_table(w.block_tables, hi))
    lens = dev32(w.seq_lens)
    q = dev16(w.q)
    msl = w.max_seq_len
    out = pa.append_decode_attention(q, dev16(w.k_new), dev16(w.v_new), kp, vp, bt, lens, msl,
                                     scale=w.scale)
    torch.cuda.synchronize()
    k_post, v_post = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                      w.seq_lens)
    assert np.array_equal(host16(kp[hi_t]), k_post) and np.array_equal(host16(vp[hi_t]), v_post)
    placed = set(hi.tolist())          # compared in full with the oracle's pools above
    for pool, name in ((kp, "k"), (vp, "v")):
        assert set(_touched_pages(pool, poison).tolist()) <= placed, \
            f"{name} pool: a page outside the batch's pages was written"
    ref = oracle.decode_attention(w.q, k_post, v_post, w.block_tables, w.seq_lens, w.scale)
    assert_close(out.cpu().numpy().astype(np.float64), ref, where="bf16 fused, pages past 4 GiB")

    def decode(kind, kw):
        if kind == "grid":
            o = pa.decode_attention(q, kp, vp, bt, lens, msl, scale=w.scale, **kw)
        elif kind == "worklist":
            o = pa.append_decode_attention_worklist(q, None, None, kp, vp, bt, lens, msl,
                                                    kw["work"], kw["pages_per_split"],
                                                    scale=w.scale)
        else:
            o = pa.decode_balanced(q, kp, vp, bt, lens, msl, kw["plan"], scale=w.scale)
        torch.cuda.synchronize()
        return o.cpu().numpy().astype(np.float64)
    _check_launches(decode, ref, w.seq_lens, total, msl, "bf16")
    del kp, vp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nbits", [8, 4])
def test_quantised_pages_past_4_gib(nbits):
    pa = _pa()
    small_pages = sum(W.pages_for(L) for L in LENS) + 7
    w = W.make_q8_batch(LENS, small_pages, 4410 + nbits, append=True, nbits=nbits)
    row = W.HEAD_DIM if nbits == 8 else W.HEAD_DIM // 2
    total, hi = _high_map(small_pages, W.NUM_KV_HEADS * W.PAGE_SIZE * row, 4420 + nbits)
    _say(f"int{nbits}: pool of {total} pages ({total * 8 * 16 * row / 2**30:.2f} GiB per code "
         f"pool), pages {hi.min()} .. {hi.max()}")
    dt = torch.int8 if nbits == 8 else torch.uint8
    code_poison = torch.tensor(-128 if nbits == 8 else 0xA5, dtype=dt, device="cuda")
    hi_t = torch.from_numpy(hi).cuda()
    kc = torch.full((total, 8, 16, row), int(code_poison), dtype=dt, device="cuda")
    vc = torch.full_like(kc, int(code_poison))
    sc = torch.full((total, 8, 2, 16), float("nan"), dtype=torch.float32, device="cuda")
    kc[hi_t] = torch.from_numpy(np.ascontiguousarray(w.k_codes)).cuda()
    vc[hi_t] = torch.from_numpy(np.ascontiguousarray(w.v_codes)).cuda()
    sc[hi_t] = torch.from_numpy(np.ascontiguousarray(w.kv_scales)).cuda()
    bt = dev32(_map_table(w.block_tables, hi))
    lens = dev32(w.seq_lens)
    q = dev16(w.q)
    msl = w.max_seq_len
    fused = pa.append_decode_attention_q8 if nbits == 8 else pa.append_decode_attention_q4
    out = fused(q, dev16(w.k_new), dev16(w.v_new), kc, vc, sc, bt, lens, msl, scale=w.scale)
    torch.cuda.synchronize()
    pools = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                 w.block_tables, w.seq_lens, nbits=nbits)
    assert np.array_equal(kc[hi_t].cpu().numpy(), pools[0])
    assert np.array_equal(vc[hi_t].cpu().numpy(), pools[1])
    assert np.array_equal(sc[hi_t].cpu().numpy().view(np.uint32), pools[2].view(np.uint32))
    placed = set(hi.tolist())          # compared in full with the oracle's pools above
    for pool, name in ((kc, "k codes"), (vc, "v codes")):
        assert set(_touched_pages(pool, code_poison).tolist()) <= placed, \
            f"{name}: a page outside the batch's pages was written"
    assert set(torch.nonzero(~torch.isnan(sc.view(total, -1)).all(dim=1)).flatten()
               .cpu().numpy().tolist()) <= placed, "scales: a page outside the batch's pages was written"
    ref = kvquant.decode_attention_q8(w.q, *pools, w.block_tables, w.seq_lens, w.scale,
                                      nbits=nbits)
    assert_close(out.cpu().numpy().astype(np.float64), ref,
                 where=f"int{nbits} fused, pages past 4 GiB")

    def decode(kind, kw):
        if kind == "grid":
            o = pa.decode_attention_q8(q, kc, vc, sc, bt, lens, msl, scale=w.scale, nbits=nbits,
                                       **kw)
        elif kind == "worklist":
            o = pa.append_decode_attention_worklist(q, None, None, kc, vc, bt, lens, msl,
                                                    kw["work"], kw["pages_per_split"],
                                                    scale=w.scale, kv_scales=sc)
        else:
            o = pa.decode_balanced(q, kc, vc, bt, lens, msl, kw["plan"], kv_scales=sc,
                                   scale=w.scale)
        torch.cuda.synchronize()
        return o.cpu().numpy().astype(np.float64)
    _check_launches(decode, ref, w.seq_lens, total, msl, f"int{nbits}",
                    int8=nbits == 8, int4=nbits == 4)
    del kc, vc, sc
    torch.cuda.empty_cache()
