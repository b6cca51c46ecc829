"""INT4 K/V pages on the GPU against the oracle.

* quantised append, append with RoPE and prefill fill at 4 bits: packed
  codes and scales bit-exact against the oracle's quantiser and packing;
* decode over INT4 pages (random packed codes and scales from the seeded
  generator, random bytes and NaN scales in every unused slot): within the
  attention tolerance of the float64 oracle over the dequantised cache, over
  split sizes, output types, edge lengths and bad metadata, with one and with
  two wavefronts per KV head (plans whose grid fits the CUs with splits of 32
  pages or more), including empty and uneven second halves;
* the fused quantise-append + decode: pools bit-identical to the two-call
  form, outputs identical to it and within tolerance of the oracle; with
  RoPE; behind 256-entry block tables; launched from a work list;
* at the full 256 x 2048 size with the planner's split size: the BF16 cache
  quantised on the GPU, every page and output against the oracle, and
  the quantisation error against BF16 attention within the oracle's
  analytic bound.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close, dev16, dev32, host16
from oracle import kvquant

pytestmark = pytest.mark.gpu

HKV, D, P, HQ = W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE, W.NUM_Q_HEADS
NB = 4


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from paged_kv_decode_07_amd import binding
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _pa():
    from paged_kv_decode_07_amd import binding as pa
    return pa


class DevQ4:
    def __init__(self, w: W.Q8Batch):
        assert w.nbits == NB
        self.h = w
        self.q = dev16(w.q)
        self.kc = torch.from_numpy(np.ascontiguousarray(w.k_codes)).cuda()
        self.vc = torch.from_numpy(np.ascontiguousarray(w.v_codes)).cuda()
        self.sc = torch.from_numpy(np.ascontiguousarray(w.kv_scales)).cuda()
        self.bt = dev32(w.block_tables)
        self.lens = dev32(w.seq_lens)
        self.k_new = dev16(w.k_new) if w.k_new is not None else None
        self.v_new = dev16(w.v_new) if w.v_new is not None else None

    def pools(self):
        torch.cuda.synchronize()
        return self.kc.cpu().numpy(), self.vc.cpu().numpy(), self.sc.cpu().numpy()


def _same_pools(got, want):
    for g, w_, name in zip(got, want, ("k codes", "v codes", "scales")):
        if name == "scales":     # compare bit patterns: NaN poison must stay where it was
            assert np.array_equal(g.view(np.uint32), w_.view(np.uint32)), name
        else:
            assert np.array_equal(g, w_), name


def _special_rows():
    """BF16 rows [6][8][64] on the 4-bit quantiser's edges."""
    rng = np.random.default_rng(1901)
    rows = W.f32_to_bf16_bits(rng.standard_normal((6, HKV, D), dtype=np.float32))
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "int4_quant_examples.json")))
    for i, r in enumerate(g["rows"]):
        vals = np.resize(np.array(r["values"], np.float32), D)
        rows[i, i % HKV] = W.f32_to_bf16_bits(vals)                  # golden rows, tiled to 64
    rows[3, 1] = 0                                                   # all-zero row
    rows[3, 2] = W.f32_to_bf16_bits(np.linspace(-1e-38, 1e-38, D, dtype=np.float32))  # tiny
    rows[4, 3] = W.f32_to_bf16_bits(np.linspace(-3e38, 2e38, D, dtype=np.float32))    # huge
    rows[5, 4] = W.f32_to_bf16_bits(np.resize(np.arange(-14, 15, dtype=np.float32) / 2, D))  # ties
    return rows


# ---------------------------------------------------------------------------
# Quantiser: append, append with RoPE, fill
# ---------------------------------------------------------------------------
def test_q4_append_bitexact():
    pa = _pa()
    lens = [1, 16, 17, 0, 2048, 33, 100, 5]
    w = W.make_q8_batch(lens, 300, 1911, append=True, nbits=NB)
    w.k_new[:6] = _special_rows()
    w.v_new[2:8] = _special_rows()
    d = DevQ4(w)
    pa.append_kv_q4(d.k_new, d.v_new, d.kc, d.vc, d.sc, d.bt, d.lens)
    want = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                w.block_tables, w.seq_lens, nbits=NB)
    _same_pools(d.pools(), want)


def test_q4_append_rope_bitexact():
    pa = _pa()
    lens = [1, 16, 17, 0, 2048, 33, 700]
    w = W.make_q8_batch(lens, 300, 1912, append=True, nbits=NB)
    cos, sin = W.rope_table()
    d = DevQ4(w)
    q_out = pa.append_kv_rope_q4(d.q, d.k_new, d.v_new, torch.from_numpy(cos).cuda(),
                                 torch.from_numpy(sin).cuda(), d.kc, d.vc, d.sc, d.bt, d.lens)
    q_ref, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    assert np.array_equal(host16(q_out), q_ref)
    want = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, k_rot, w.v_new,
                                w.block_tables, w.seq_lens, nbits=NB)
    _same_pools(d.pools(), want)


@pytest.mark.parametrize("start,count", [(0, 1), (0, 37), (5, 16), (16, 17), (0, 2048), (1000, 1048)])
def test_q4_fill_bitexact(start, count):
    pa = _pa()
    rng = np.random.default_rng(start * 17 + count)
    pages = 200
    kc, vc, sc = (rng.integers(0, 256, (pages, HKV, P, D // 2), dtype=np.uint8),
                  rng.integers(0, 256, (pages, HKV, P, D // 2), dtype=np.uint8),
                  np.full((pages, HKV, 2, P), np.nan, np.float32))
    row = np.full(128, -1, np.int32)
    n = W.pages_for(start + count)
    row[:n] = rng.permutation(pages)[:n]
    kr, vr = W.random_rows(rng, count), W.random_rows(rng, count)
    if count >= 6:
        kr[:6] = _special_rows()
    dk, dv, ds = (torch.from_numpy(a.copy()).cuda() for a in (kc, vc, sc))
    pa.fill_kv_q4(dev16(kr), dev16(vr), dev32(row), start, dk, dv, ds)
    torch.cuda.synchronize()
    want = kvquant.fill_kv_q8(kc, vc, sc, kr, vr, row, start, nbits=NB)
    _same_pools((dk.cpu().numpy(), dv.cpu().numpy(), ds.cpu().numpy()), want)


# ---------------------------------------------------------------------------
# Decode over INT4 pages
# ---------------------------------------------------------------------------
EDGE = [1, 2, 15, 16, 17, 32, 33, 100, 2047, 2048, 0]


def _decode(d, ps=0, out_dtype=torch.float32, max_seq_len=None):
    pa = _pa()
    msl = d.h.max_seq_len if max_seq_len is None else max_seq_len
    out = pa.decode_attention_q4(d.q, d.kc, d.vc, d.sc, d.bt, d.lens, msl, scale=d.h.scale,
                                 out_dtype=out_dtype, pages_per_split=ps)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _ref(w, sequences=None, pools=None, q=None):
    kc, vc, sc = pools if pools is not None else (w.k_codes, w.v_codes, w.kv_scales)
    return kvquant.decode_attention_q8(w.q if q is None else q, kc, vc, sc, w.block_tables,
                                       w.seq_lens, w.scale, sequences=sequences, nbits=NB)


@pytest.mark.parametrize("pages_per_split", [0, 1, 3, 16, 128])
def test_q4_decode_edge_lengths(pages_per_split):
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 1921, nbits=NB)
    got = _decode(DevQ4(w), pages_per_split)
    assert_close(got, _ref(w), where=f"q4 edge ps={pages_per_split}")
    assert np.all(got[-1] == 0.0)


def test_q4_two_waves_per_head_uneven_halves():
    """Plans whose grid (batch x splits) fits the CUs and whose splits hold 32 pages or more run
    two wavefronts per KV head: each streams half of its split's pages and the two states merge
    through LDS.  Sequences of 1, 2, 17, 33 and 63 pages under 32- and 33-page splits give
    empty, single-page, even and uneven second halves.  A block-table entry outside the pool
    that only the second wavefront reads must still turn that sequence's outputs into NaN."""
    lens = [1, 16, 17 * 16, 33 * 16 - 5, 63 * 16, 2048, 0]
    w = W.make_q8_batch(lens, sum(W.pages_for(L) for L in lens) + 5, 1931, nbits=NB)
    d = DevQ4(w)
    ref = _ref(w)
    for ps in (32, 33, 128):
        assert_close(_decode(d, ps), ref, where=f"q4 two waves ps={ps}")
    # sequence 4 (63 pages in one 128-page split): halves 0..31 and 32..62
    bt = w.block_tables.copy()
    bt[4, 40] = w.k_codes.shape[0] + 3
    d.bt = dev32(bt)
    got = _decode(d, 128)
    assert np.all(np.isnan(got[4]))
    others = [0, 1, 2, 3, 5, 6]
    assert_close(got[others], ref[others], where="q4 two waves, other sequences")


def test_q4_decode_bf16_out():
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 1922, nbits=NB)
    got = _decode(DevQ4(w), 4, out_dtype=torch.bfloat16)
    assert_close(got, _ref(w), bf16_out=True, where="q4 bf16 out")


def test_q4_decode_random_lengths_identity_placement():
    lens = W.workload_seq_lens(3)
    w = W.make_q8_batch(lens, 8192, 1923, placement="identity", nbits=NB)
    got = _decode(DevQ4(w))
    assert_close(got, _ref(w), where="q4 batch 64 identity")


def test_q4_decode_sharp_scores():
    """Large scale factors: one token dominates each head, so the output is
    close to one dequantised V row and the code bias must cancel exactly."""
    w = W.make_q8_batch([700, 16, 1], 64, 1924, nbits=NB)
    w.scale = 2.0
    got = _decode(DevQ4(w), 8)
    assert_close(got, _ref(w), where="q4 sharp scores")


def test_q4_decode_bad_metadata():
    w = W.make_q8_batch([40, 40, 40, 0], 16, 1925, nbits=NB)
    w.block_tables[1, 1] = 16                    # page id past the pool
    w.block_tables[2, 0] = -3
    got = _decode(DevQ4(w))
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.all(got[3] == 0)
    assert_close(got[:1], _ref(w, sequences=[0])[:1], where="q4 good row beside bad ones")
    w2 = W.make_q8_batch([40, 50], 16, 1926, nbits=NB)
    got2 = _decode(DevQ4(w2), max_seq_len=45)    # sequence 1 exceeds the declared bound
    assert np.all(np.isnan(got2[1]))
    assert_close(got2[:1], _ref(w2, sequences=[0])[:1], where="q4 length bound")


# ---------------------------------------------------------------------------
# Fused quantise-append + decode
# ---------------------------------------------------------------------------
def _fused(d, ps=0, rope=None, out_dtype=torch.float32):
    pa = _pa()
    kw = {}
    if rope is not None:
        kw = dict(rope_cos=torch.from_numpy(rope[0]).cuda(), rope_sin=torch.from_numpy(rope[1]).cuda())
    out = pa.append_decode_attention_q4(d.q, d.k_new, d.v_new, d.kc, d.vc, d.sc, d.bt, d.lens,
                                        d.h.max_seq_len, scale=d.h.scale, out_dtype=out_dtype,
                                        pages_per_split=ps, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _appended_pools(w, k_rows=None):
    return kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales,
                                w.k_new if k_rows is None else k_rows, w.v_new,
                                w.block_tables, w.seq_lens, nbits=NB)


@pytest.mark.parametrize("pages_per_split", [0, 1, 3, 16, 128])
def test_q4_fused_matches_two_call_and_oracle(pages_per_split):
    pa = _pa()
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 1931, append=True, nbits=NB)
    w.k_new[:6] = _special_rows()
    a = DevQ4(w)
    pa.append_kv_q4(a.k_new, a.v_new, a.kc, a.vc, a.sc, a.bt, a.lens)
    two = _decode(a, pages_per_split)
    f = DevQ4(w)
    fused = _fused(f, pages_per_split)
    _same_pools(f.pools(), a.pools())
    assert np.array_equal(fused, two), "fused output differs from append + decode"
    pools = _appended_pools(w)
    _same_pools(f.pools(), pools)
    assert_close(fused, _ref(w, pools=pools), where=f"q4 fused ps={pages_per_split}")


@pytest.mark.parametrize("pages_per_split", [2, 128])
def test_q4_fused_bf16_out(pages_per_split):
    # 2-page splits: one wavefront per KV head; 128-page splits: two
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 1933, append=True, nbits=NB)
    got = _fused(DevQ4(w), pages_per_split, out_dtype=torch.bfloat16)
    assert_close(got, _ref(w, pools=_appended_pools(w)), bf16_out=True,
                 where=f"q4 fused bf16 out ps={pages_per_split}")


@pytest.mark.parametrize("pages_per_split", [3, 64])
def test_q4_fused_rope_matches_oracle(pages_per_split):
    # 3-page splits: one wavefront per KV head; 64-page splits (22 work-groups): two
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 1932, append=True, nbits=NB)
    cos, sin = W.rope_table()
    f = DevQ4(w)
    got = _fused(f, pages_per_split, rope=(cos, sin))
    q_rot, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    pools = _appended_pools(w, k_rows=k_rot)
    _same_pools(f.pools(), pools)
    assert_close(got, _ref(w, pools=pools, q=q_rot), where=f"q4 fused rope ps={pages_per_split}")


@pytest.mark.parametrize("pages_per_split", [0, 256])
def test_q4_fused_4096_token_tables(pages_per_split):
    """INT4 pages behind 256-entry block tables, splits up to 256 pages."""
    lens = [4096, 3999, 33, 0, 1]
    w = W.make_q8_batch(lens, sum(W.pages_for(L) for L in lens) + 5, 4099, append=True,
                        max_blocks=256, nbits=NB)
    f = DevQ4(w)
    fused = _fused(f, pages_per_split)
    pools = _appended_pools(w)
    _same_pools(f.pools(), pools)
    assert_close(fused, _ref(w, pools=pools), where=f"q4 4096-token tables ps={pages_per_split}")


def test_q4_worklist_matches_grid():
    """The work-list launch gives the grid launch's pools and outputs bit for bit."""
    pa = _pa()
    lens = W.workload_seq_lens(5)[:96]
    w = W.make_q8_batch(lens, sum(W.pages_for(L) for L in lens) + 7, 1941, append=True, nbits=NB)
    work, ps, _ = pa.decode_worklist(w.seq_lens, w.num_pages, int4=True)
    g = DevQ4(w)
    grid = _fused(g, ps)
    f = DevQ4(w)
    out = pa.append_decode_attention_worklist(f.q, f.k_new, f.v_new, f.kc, f.vc, f.bt, f.lens,
                                              w.max_seq_len, dev32(work), ps, scale=w.scale,
                                              kv_scales=f.sc)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    _same_pools(f.pools(), g.pools())
    assert np.array_equal(got, grid)
    assert_close(got, _ref(w, pools=_appended_pools(w)), where="q4 work list")


# ---------------------------------------------------------------------------
# Full size, as the benchmark runs it
# ---------------------------------------------------------------------------
def test_q4_full_batch256_len2048_bench_configuration():
    """BF16 workload (256 x 2048, append) quantised to 4 bits on the GPU page by
    page, then the fused INT4 step with the planner's split size."""
    pa = _pa()
    w = W.make_workload(4, append=True)
    npg = w.num_pages
    k16, v16 = dev16(w.k_pool), dev16(w.v_pool)
    kc, vc, sc = pa.new_q4_pools(npg)
    ident = dev32(np.arange(npg, dtype=np.int32))
    pa.fill_kv_q4(k16.view(npg * P, HKV, D), v16.view(npg * P, HKV, D), ident, 0, kc, vc, sc)
    ps, _ = pa.decode_plan_lengths_q4(w.seq_lens, npg)
    out = pa.append_decode_attention_q4(dev16(w.q), dev16(w.k_new), dev16(w.v_new), kc, vc, sc,
                                        dev32(w.block_tables), dev32(w.seq_lens), w.max_seq_len,
                                        scale=w.scale, pages_per_split=ps)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    qf = oracle.bf16_bits_to_f64(w.q)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        pages = w.block_tables[b, :W.pages_for(L)]
        kr = w.k_pool[pages].reshape(-1, HKV, D)[:L].copy()
        vr = w.v_pool[pages].reshape(-1, HKV, D)[:L].copy()
        kr[L - 1], vr[L - 1] = w.k_new[b], w.v_new[b]
        kq, ks = kvquant.quantize_rows(kr, NB)
        vq, vs = kvquant.quantize_rows(vr, NB)
        sel = torch.from_numpy(pages).long().cuda()
        gk = np.swapaxes(kc[sel].cpu().numpy(), 1, 2).reshape(-1, HKV, D // 2)[:L]
        assert np.array_equal(gk, kvquant.pack_q4(kq))
        gs = sc[sel].cpu().numpy()
        gks = np.transpose(gs[:, :, 0, :], (0, 2, 1)).reshape(-1, HKV)[:L]
        assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
        K, V = kvquant.dequantize(kq, ks), kvquant.dequantize(vq, vs)
        Kb, Vb = oracle.bf16_bits_to_f64(kr), oracle.bf16_bits_to_f64(vr)
        for h in range(HQ):
            g = h // (HQ // HKV)
            o, _, _ = oracle.attention_one_query(qf[b, h], K[:, g], V[:, g], w.scale)
            assert_close(got[b, h][None], o[None], where=f"q4 full b={b} h={h}")
            ob, _, _ = oracle.attention_one_query(qf[b, h], Kb[:, g], Vb[:, g], w.scale)
            bound = kvquant.quantisation_error_bound(qf[b, h], Kb[:, g], K[:, g], Vb[:, g],
                                                     V[:, g], w.scale)
            assert np.all(np.abs(got[b, h] - ob) <= bound + 2e-3), (b, h)
