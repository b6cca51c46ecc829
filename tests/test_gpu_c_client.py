"""The library driven from C++ alone: a host program (tests/c_client) that
allocates with hipMalloc, calls the header's pa_append_decode_attention (or
its INT8 and INT4 forms, the balanced launch over a plan it builds from the
host lengths, or the allocation-free step) on the default stream and writes
the results back to files.  No Python binding or torch tensor takes part in the step; the outputs
are checked against the oracle as in the binding's parity tests (pools
bit-exact, attention within the FP32 bound)."""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import ATOL_F32
from oracle import kvquant

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "paged_kv_decode_07_amd", "_lib", "decode_client")


@pytest.mark.parametrize("lens,pps,launch,heads", [
    ([37, 1, 200, 16, 0, 513], 0, 0, 8), ([2048] * 3, 8, 0, 8),
    ([37, 1, 200, 16, 0, 513], 0, 1, 8), ([2048] * 3, 0, 1, 1),
    ([37, 1, 200, 16, 0, 513], 4, 2, 8)],
    ids=["ragged-auto", "long-split8", "balanced-ragged", "balanced-long-1-head-lanes",
         "noalloc-ragged-split4"])
def test_c_client_step_matches_oracle(tmp_path, lens, pps, launch, heads):
    if not os.path.exists(CLIENT):
        pytest.fail("decode_client is not built (build the library and the client first)")
    pages = sum(W.pages_for(L) for L in lens) + 5
    w = W.make_batch(lens, pages, seed=2100 + len(lens), append=True)
    B = len(lens)
    rng = np.random.default_rng(2200 + B)
    k_new, v_new = W.random_rows(rng, B), W.random_rows(rng, B)
    max_len = max(lens)
    for name, arr in (("q", w.q), ("k_new", k_new), ("v_new", v_new), ("k_pool", w.k_pool),
                      ("v_pool", w.v_pool), ("bt", w.block_tables), ("lens", w.seq_lens)):
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(
        f"{B} {pages} {W.MAX_BLOCKS} {max_len} {pps} 16 {launch} {heads}\n")
    print(f"c_client: lens {lens} pps {pps} launch {launch} heads {heads}", flush=True)
    res = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"client exit {res.returncode}: {res.stdout}{res.stderr}"

    k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, k_new, v_new, w.block_tables, w.seq_lens)
    k_out = np.fromfile(tmp_path / "k_pool_out.bin", np.uint16).reshape(k_ref.shape)
    v_out = np.fromfile(tmp_path / "v_pool_out.bin", np.uint16).reshape(v_ref.shape)
    assert np.array_equal(k_out, k_ref) and np.array_equal(v_out, v_ref)
    ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale)
    out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(ref.shape).astype(np.float64)
    err = float(np.max(np.abs(out - ref)))
    assert err <= ATOL_F32, err
    assert np.all(out[w.seq_lens == 0] == 0)          # an idle slot's rows are zero


@pytest.mark.parametrize("bits,lens,pps,launch", [(8, [37, 1, 200, 16, 0, 513], 0, 0),
                                                  (4, [37, 1, 200, 16, 0, 513], 0, 0),
                                                  (4, [2048] * 3, 64, 0),
                                                  (8, [37, 1, 200, 16, 0, 513], 0, 1),
                                                  (4, [2048, 17, 1000], 0, 1)],
                         ids=["int8-ragged-auto", "int4-ragged-auto", "int4-long-split64",
                              "int8-balanced", "int4-balanced"])
def test_c_client_quantised_step_matches_oracle(tmp_path, bits, lens, pps, launch):
    if not os.path.exists(CLIENT):
        pytest.fail("decode_client is not built (build the library and the client first)")
    pages = sum(W.pages_for(L) for L in lens) + 5
    w = W.make_q8_batch(lens, pages, 2300 + bits + len(lens), append=True, nbits=bits)
    B = len(lens)
    for name, arr in (("q", w.q), ("k_new", w.k_new), ("v_new", w.v_new), ("k_pool", w.k_codes),
                      ("v_pool", w.v_codes), ("scales", w.kv_scales), ("bt", w.block_tables),
                      ("lens", w.seq_lens)):
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(
        f"{B} {pages} {W.MAX_BLOCKS} {max(lens)} {pps} {bits} {launch}\n")
    print(f"c_client: {bits}-bit pages, lens {lens} pps {pps} launch {launch}", flush=True)
    res = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"client exit {res.returncode}: {res.stdout}{res.stderr}"

    kc, vc, sc = kvquant.append_kv_q8(w.k_codes, w.v_codes, w.kv_scales, w.k_new, w.v_new,
                                      w.block_tables, w.seq_lens, nbits=bits)
    k_out = np.fromfile(tmp_path / "k_pool_out.bin", kc.dtype).reshape(kc.shape)
    v_out = np.fromfile(tmp_path / "v_pool_out.bin", vc.dtype).reshape(vc.shape)
    s_out = np.fromfile(tmp_path / "scales_out.bin", np.uint32).reshape(sc.shape)
    assert np.array_equal(k_out, kc) and np.array_equal(v_out, vc)
    assert np.array_equal(s_out, sc.view(np.uint32))             # NaN poison kept bit for bit
    ref = kvquant.decode_attention_q8(w.q, kc, vc, sc, w.block_tables, w.seq_lens, w.scale,
                                      nbits=bits)
    out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(ref.shape).astype(np.float64)
    err = float(np.max(np.abs(out - ref)))
    assert err <= ATOL_F32, err
    assert np.all(out[w.seq_lens == 0] == 0)
