"""INT8 K/V pages on the GPU against the oracle.

* quantised append, append with RoPE and prefill fill: codes and scales
  bit-exact against the oracle's quantiser (same FP32 decisions);
* decode over INT8 pages (random codes and scales from the seeded generator,
  NaN scales in every unused slot): within the attention tolerance of the
  float64 oracle over the dequantised cache, over split sizes, output types,
  edge lengths and bad metadata;
* the fused quantise-append + decode: pools bit-identical to the two-call
  form, outputs identical to it and within tolerance of the oracle;
* at the full 256 x 2048 size, in the launch configuration the benchmark
  times: the BF16 cache quantised on the GPU, every page and output
  against the oracle, and the quantisation error against BF16 attention
  within the oracle's analytic bound.
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


class DevQ8:
    def __init__(self, w: W.Q8Batch):
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
    """BF16 rows [6][8][64] on the quantiser's edges."""
    rng = np.random.default_rng(901)
    rows = W.f32_to_bf16_bits(rng.standard_normal((6, HKV, D), dtype=np.float32))
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "int8_quant_examples.json")))
    for i, r in enumerate(g["rows"]):
        vals = np.resize(np.array(r["values"], np.float32), D)
        rows[i, i % HKV] = W.f32_to_bf16_bits(vals)                  # golden rows, tiled to 64
    rows[3, 1] = 0                                                   # all-zero row
    rows[3, 2] = W.f32_to_bf16_bits(np.linspace(-1e-38, 1e-38, D, dtype=np.float32))  # tiny
    rows[4, 3] = W.f32_to_bf16_bits(np.linspace(-3e38, 2e38, D, dtype=np.float32))    # huge
    rows[5, 4] = W.f32_to_bf16_bits(np.arange(D, dtype=np.float32) - 31.5)              # ties
    return rows


# ---------------------------------------------------------------------------
# Quantiser: append, append with RoPE, fill
# ---------------------------------------------------------------------------
def test_q8_append_bitexact():
    pa = _pa()
    lens = [1, 16, 17, 0, 2048, 33, 100, 5]
    w = W.make_q8_batch(lens, 300, 911, append=True)
    w.k_new[:6] = _special_rows()
    w.v_new[2:8] = _special_rows()
    d = DevQ8(w)
    pa.append_kv_q8(d.k_new, d.v_new, d.kc, d.vc, d.sc, d.bt, d.lens)
    want = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                w.block_tables, w.seq_lens)
    _same_pools(d.pools(), want)


def test_q8_append_rope_bitexact():
    pa = _pa()
    lens = [1, 16, 17, 0, 2048, 33, 700]
    w = W.make_q8_batch(lens, 300, 912, append=True)
    cos, sin = W.rope_table()
    d = DevQ8(w)
    q_out = pa.append_kv_rope_q8(d.q, d.k_new, d.v_new, torch.from_numpy(cos).cuda(),
                                 torch.from_numpy(sin).cuda(), d.kc, d.vc, d.sc, d.bt, d.lens)
    q_ref, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    assert np.array_equal(host16(q_out), q_ref)
    want = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, k_rot, w.v_new,
                                w.block_tables, w.seq_lens)
    _same_pools(d.pools(), want)


@pytest.mark.parametrize("start,count", [(0, 1), (0, 37), (5, 16), (16, 17), (0, 2048), (1000, 1048)])
def test_q8_fill_bitexact(start, count):
    pa = _pa()
    rng = np.random.default_rng(start * 13 + count)
    pages = 200
    kc, vc, sc = (rng.integers(-128, 128, (pages, HKV, P, D), dtype=np.int8),
                  rng.integers(-128, 128, (pages, HKV, P, D), dtype=np.int8),
                  np.full((pages, HKV, 2, P), np.nan, np.float32))
    row = np.full(128, -1, np.int32)
    n = W.pages_for(start + count)
    row[:n] = rng.permutation(pages)[:n]
    kr, vr = W.random_rows(rng, count), W.random_rows(rng, count)
    if count >= 6:
        kr[:6] = _special_rows()
    dk, dv, ds = (torch.from_numpy(a.copy()).cuda() for a in (kc, vc, sc))
    pa.fill_kv_q8(dev16(kr), dev16(vr), dev32(row), start, dk, dv, ds)
    torch.cuda.synchronize()
    want = kvquant.fill_kv_q8(kc, vc, sc, kr, vr, row, start)
    _same_pools((dk.cpu().numpy(), dv.cpu().numpy(), ds.cpu().numpy()), want)


# ---------------------------------------------------------------------------
# Decode over INT8 pages
# ---------------------------------------------------------------------------
EDGE = [1, 2, 15, 16, 17, 32, 33, 100, 2047, 2048, 0]


def _decode(d, ps=0, out_dtype=torch.float32, max_seq_len=None):
    pa = _pa()
    msl = d.h.max_seq_len if max_seq_len is None else max_seq_len
    out = pa.decode_attention_q8(d.q, d.kc, d.vc, d.sc, d.bt, d.lens, msl, scale=d.h.scale,
                                 out_dtype=out_dtype, pages_per_split=ps)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _ref(w, sequences=None, pools=None):
    kc, vc, sc = pools if pools is not None else (w.k_codes, w.v_codes, w.kv_scales)
    return kvquant.decode_attention_q8(w.q, kc, vc, sc, w.block_tables, w.seq_lens, w.scale,
                                       sequences=sequences)


@pytest.mark.parametrize("pages_per_split", [0, 1, 3, 16, 128])
def test_q8_decode_edge_lengths(pages_per_split):
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 921)
    got = _decode(DevQ8(w), pages_per_split)
    assert_close(got, _ref(w), where=f"q8 edge ps={pages_per_split}")
    assert np.all(got[-1] == 0.0)


def test_q8_decode_bf16_out():
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 922)
    got = _decode(DevQ8(w), 4, out_dtype=torch.bfloat16)
    assert_close(got, _ref(w), bf16_out=True, where="q8 bf16 out")


def test_q8_decode_random_lengths_identity_placement():
    lens = W.workload_seq_lens(3)
    w = W.make_q8_batch(lens, 8192, 923, placement="identity")
    d = DevQ8(w)
    got = _decode(d)
    assert_close(got, _ref(w), where="q8 batch 64 identity")


def test_q8_decode_bad_metadata():
    w = W.make_q8_batch([40, 40, 40, 0], 16, 924)
    w.block_tables[1, 1] = 16                    # page id past the pool
    w.block_tables[2, 0] = -3
    d = DevQ8(w)
    got = _decode(d)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.all(got[3] == 0)
    assert_close(got[:1], _ref(w, sequences=[0])[:1], where="q8 good row beside bad ones")
    w2 = W.make_q8_batch([40, 50], 16, 925)
    d2 = DevQ8(w2)
    got2 = _decode(d2, max_seq_len=45)          # sequence 1 exceeds the declared bound
    assert np.all(np.isnan(got2[1]))
    assert_close(got2[:1], _ref(w2, sequences=[0])[:1], where="q8 length bound")


# ---------------------------------------------------------------------------
# Fused quantise-append + decode
# ---------------------------------------------------------------------------
def _fused(d, ps=0, rope=None, out_dtype=torch.float32):
    pa = _pa()
    kw = {}
    if rope is not None:
        kw = dict(rope_cos=torch.from_numpy(rope[0]).cuda(), rope_sin=torch.from_numpy(rope[1]).cuda())
    out = pa.append_decode_attention_q8(d.q, d.k_new, d.v_new, d.kc, d.vc, d.sc, d.bt, d.lens,
                                        d.h.max_seq_len, scale=d.h.scale, out_dtype=out_dtype,
                                        pages_per_split=ps, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("pages_per_split", [0, 1, 3, 16, 128])
def test_q8_fused_matches_two_call_and_oracle(pages_per_split):
    pa = _pa()
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 931, append=True)
    w.k_new[:6] = _special_rows()
    a = DevQ8(w)
    pa.append_kv_q8(a.k_new, a.v_new, a.kc, a.vc, a.sc, a.bt, a.lens)
    two = _decode(a, pages_per_split)
    f = DevQ8(w)
    fused = _fused(f, pages_per_split)
    _same_pools(f.pools(), a.pools())
    assert np.array_equal(fused, two), "fused output differs from append + decode"
    pools = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                 w.block_tables, w.seq_lens)
    _same_pools(f.pools(), pools)
    assert_close(fused, _ref(w, pools=pools), where=f"q8 fused ps={pages_per_split}")


def test_q8_fused_rope_matches_oracle():
    w = W.make_q8_batch(EDGE, sum(W.pages_for(L) for L in EDGE) + 9, 932, append=True)
    cos, sin = W.rope_table()
    f = DevQ8(w)
    got = _fused(f, 3, rope=(cos, sin))
    q_rot, k_rot = oracle.rope.rope_new_token(w.q, w.k_new, w.seq_lens, cos, sin)
    pools = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, k_rot, w.v_new,
                                 w.block_tables, w.seq_lens)
    _same_pools(f.pools(), pools)
    ref = kvquant.decode_attention_q8(q_rot, *pools, w.block_tables, w.seq_lens, w.scale)
    assert_close(got, ref, where="q8 fused rope")


# ---------------------------------------------------------------------------
# Full size, as the benchmark runs it
# ---------------------------------------------------------------------------
def test_q8_full_batch256_len2048_bench_configuration():
    """BF16 workload (256 x 2048, append) quantised on the GPU page by page,
    then the fused INT8 step with the planner's split size."""
    pa = _pa()
    w = W.make_workload(4, append=True)
    npg = w.num_pages
    k16, v16 = dev16(w.k_pool), dev16(w.v_pool)
    kc, vc, sc = pa.new_q8_pools(npg)
    ident = dev32(np.arange(npg, dtype=np.int32))
    # every slot of every page, as one sequence over an identity table
    pa.fill_kv_q8(k16.view(npg * P, HKV, D), v16.view(npg * P, HKV, D), ident, 0, kc, vc, sc)
    ps, _ = pa.decode_plan_lengths_q8(w.seq_lens, npg)
    out = pa.append_decode_attention_q8(dev16(w.q), dev16(w.k_new), dev16(w.v_new), kc, vc, sc,
                                        dev32(w.block_tables), dev32(w.seq_lens), w.max_seq_len,
                                        scale=w.scale, pages_per_split=ps)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    qf = oracle.bf16_bits_to_f64(w.q)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        pages = w.block_tables[b, :W.pages_for(L)]
        # logical rows of the sequence (the held-back token appended)
        kr = w.k_pool[pages].reshape(-1, HKV, D)[:L].copy()
        vr = w.v_pool[pages].reshape(-1, HKV, D)[:L].copy()
        kr[L - 1], vr[L - 1] = w.k_new[b], w.v_new[b]
        kq, ks = kvquant.quantize_rows(kr)
        vq, vs = kvquant.quantize_rows(vr)
        # the pages on the GPU hold exactly the oracle's codes and scales
        gk = np.swapaxes(kc[torch.from_numpy(pages).long().cuda()].cpu().numpy(), 1, 2)
        gk = gk.reshape(-1, HKV, D)[:L]                                    # [token][head][dim]
        gs = sc[torch.from_numpy(pages).long().cuda()].cpu().numpy()       # [n][8][2][16]
        assert np.array_equal(gk, kq)
        gks = np.transpose(gs[:, :, 0, :], (0, 2, 1)).reshape(-1, HKV)[:L]
        assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
        K, V = kvquant.dequantize(kq, ks), kvquant.dequantize(vq, vs)
        Kb, Vb = oracle.bf16_bits_to_f64(kr), oracle.bf16_bits_to_f64(vr)
        for h in range(HQ):
            g = h // (HQ // HKV)
            o, _, _ = oracle.attention_one_query(qf[b, h], K[:, g], V[:, g], w.scale)
            assert_close(got[b, h][None], o[None], where=f"q8 full b={b} h={h}")
            ob, _, _ = oracle.attention_one_query(qf[b, h], Kb[:, g], Vb[:, g], w.scale)
            bound = kvquant.quantisation_error_bound(qf[b, h], Kb[:, g], K[:, g], Vb[:, g],
                                                     V[:, g], w.scale)
            assert np.all(np.abs(got[b, h] - ob) <= bound + 2e-3), (b, h)


@pytest.mark.parametrize("pages_per_split", [0, 256])
def test_q8_fused_4096_token_tables(pages_per_split):
    """INT8 pages behind 256-entry block tables, splits up to 256 pages."""
    lens = [4096, 3999, 33, 0, 1]
    w = W.make_q8_batch(lens, sum(W.pages_for(L) for L in lens) + 5, 4098, append=True,
                        max_blocks=256)
    f = DevQ8(w)
    fused = _fused(f, pages_per_split)
    pools = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                 w.block_tables, w.seq_lens)
    _same_pools(f.pools(), pools)
    assert_close(fused, _ref(w, pools=pools), where=f"q8 4096-token tables ps={pages_per_split}")
