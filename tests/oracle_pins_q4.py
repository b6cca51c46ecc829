"""Pins for the INT4 K/V page oracle (hand-worked values, brute force, exact cases, a bound).

Each pin takes the oracle's kvquant module (or a copy with a planted
mistake).  What fixes the expected values:

* the hand-worked rows of ``golden/int4_quant_examples.json`` (the pages'
  symmetric quantiser at 4 bits with power-of-two scales, ties to even, and
  the packing of two codes per byte);
* brute force: every code is the integer in [-8, 7] nearest the FP32
  quotient, with exact rational comparisons;
* invariants (the largest magnitude maps to +-7, the reconstruction error is
  at most half a scale), and packing round trips over every byte;
* lossless cases: codes in [-7, 7] times a power of two quantise without
  error, so attention over INT4 pages equals the BF16 oracle's;
* the analytic bound on how far quantisation moves the attention output.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads as W

HKV, D, P, HQ = W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE, W.NUM_Q_HEADS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_quant_examples.json")


def _bits(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def empty_q4_pools(pages):
    return (np.full((pages, HKV, P, D // 2), 0x88, np.uint8),
            np.full((pages, HKV, P, D // 2), 0x88, np.uint8),
            np.zeros((pages, HKV, 2, P), np.float32))


def exact_grid_rows_q4(rng, n):
    """``[n][Hkv][D]`` BF16 rows that INT4 holds exactly: codes in [-7, 7] (one
    of them +-7) times 2^e, e in -4..1, per (token, head) row."""
    codes = rng.integers(-7, 8, size=(n, HKV, D))
    pick = rng.integers(0, D, size=(n, HKV))
    sign = rng.choice([-1, 1], size=(n, HKV))
    np.put_along_axis(codes, pick[..., None], (7 * sign)[..., None], axis=-1)
    e = rng.integers(-4, 2, size=(n, HKV, 1)).astype(np.float64)
    return _bits(codes * np.exp2(e))


def pin_q4_golden_rows(kq):
    g = json.load(open(GOLDEN))
    rows = np.array([r["values"] for r in g["rows"]], dtype=np.float32)
    codes, scale = kq.quantize_rows(_bits(rows), 4)
    assert np.array_equal(scale.astype(np.float64), [r["scale"] for r in g["rows"]])
    assert np.array_equal(codes.astype(np.int64), np.array([r["codes"] for r in g["rows"]]))
    assert np.array_equal(kq.pack_q4(codes).astype(np.int64), np.array([r["packed"] for r in g["rows"]]))


def pin_q4_brute_force_nearest_code(kq):
    rng = np.random.default_rng(711)
    x = W.random_rows(rng, 3)[:, :, :16]
    codes, scale = kq.quantize_rows(x, 4)
    xf = oracle.bf16_bits_to_f64(x)
    for idx in np.ndindex(*x.shape[:-1]):
        s = np.float32(scale[idx])
        amax = Fraction(float(np.max(np.abs(xf[idx]))))
        assert abs(Fraction(float(s)) - amax / 7) <= abs(Fraction(float(np.nextafter(s, np.inf))) - amax / 7)
        assert abs(Fraction(float(s)) - amax / 7) <= abs(Fraction(float(np.nextafter(s, -np.inf))) - amax / 7)
        for j in range(x.shape[-1]):
            r = Fraction(float(np.float32(np.float32(xf[idx][j]) / s)))
            best = min(range(-8, 8), key=lambda c: (abs(r - c), c % 2))
            assert int(codes[idx][j]) == best, (idx, j)


def pin_q4_invariants(kq):
    rng = np.random.default_rng(712)
    x = W.random_rows(rng, 64)
    x[3, 5] = 0
    codes, scale = kq.quantize_rows(x, 4)
    xf = oracle.bf16_bits_to_f64(x)
    amax = np.max(np.abs(xf), axis=-1)
    live = amax > 0
    assert np.all(np.abs(codes.astype(np.int64)) <= 7)
    assert np.array_equal(np.max(np.abs(codes.astype(np.int64)), axis=-1)[live], np.full(live.sum(), 7))
    s = scale.astype(np.float64)
    assert np.all(np.abs(7 * s - amax) <= amax * 2.0 ** -23)
    err = np.abs(xf - codes * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 2.0 ** -16))
    assert scale[3, 5] == 0 and not np.any(codes[3, 5])


def pin_q4_packing_round_trip(kq):
    every = np.arange(256, dtype=np.uint8)
    codes = kq.unpack_q4(every[None, :])[0]               # 512 codes
    assert np.array_equal(kq.pack_q4(codes), every)
    lo, hi = codes[0::2].astype(np.int64), codes[1::2].astype(np.int64)
    assert np.array_equal(lo, (every & 15).astype(np.int64) - 8)
    assert np.array_equal(hi, (every >> 4).astype(np.int64) - 8)
    pairs = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8).reshape(1, -1)
    assert np.array_equal(kq.unpack_q4(kq.pack_q4(pairs)), pairs)


def pin_q4_append_touches_one_slot(kq):
    rng = np.random.default_rng(713)
    pages = 12
    kc, vc, sc = empty_q4_pools(pages)
    kc[:] = rng.integers(0, 256, kc.shape)
    vc[:] = rng.integers(0, 256, vc.shape)
    sc[:] = rng.random(sc.shape, dtype=np.float32)
    bt = np.array([[7, 2, 9], [4, 0, 1], [3, 5, 6]], np.int32)
    lens = np.array([17, 0, 48], np.int32)
    kn, vn = W.random_rows(rng, 3), W.random_rows(rng, 3)
    k2, v2, s2 = kq.append_kv_q8(kc, vc, sc, kn, vn, bt, lens, nbits=4)
    changed = {(int(p), int(t)) for p, t in zip(*np.nonzero(np.any(k2 != kc, axis=(1, 3))))}
    assert changed <= {(2, 0), (6, 15)}
    for b, (page, slot) in ((0, (2, 0)), (2, (6, 15))):
        ck, skk = kq.quantize_rows(kn[b], 4)
        cv, svv = kq.quantize_rows(vn[b], 4)
        assert np.array_equal(k2[page, :, slot], kq.pack_q4(ck))
        assert np.array_equal(v2[page, :, slot], kq.pack_q4(cv))
        assert np.array_equal(s2[page, :, 0, slot], skk) and np.array_equal(s2[page, :, 1, slot], svv)
    mask = np.ones(sc.shape, bool)
    mask[2, :, :, 0] = False
    mask[6, :, :, 15] = False
    assert np.array_equal(s2[mask], sc[mask])


def pin_q4_fill_equals_appends(kq):
    rng = np.random.default_rng(714)
    pages, T, start = 10, 37, 5
    kc, vc, sc = empty_q4_pools(pages)
    row = rng.permutation(pages)[: W.pages_for(start + T)].astype(np.int32)
    kr, vr = W.random_rows(rng, T), W.random_rows(rng, T)
    f = kq.fill_kv_q8(kc, vc, sc, kr, vr, row, start, nbits=4)
    a = (kc, vc, sc)
    for j in range(T):
        a = kq.append_kv_q8(*a, kr[j:j + 1], vr[j:j + 1], row[None, :],
                            np.array([start + j + 1], np.int32), nbits=4)
    for x, y in zip(f, a):
        assert np.array_equal(x, y)


def _fill_both_q4(kq, rng, lens, pages, rows_fn):
    B = len(lens)
    mb = max(W.pages_for(int(L)) for L in lens) + 1
    perm = rng.permutation(pages)
    bt = np.full((B, mb), -1, np.int32)
    k16 = np.full((pages, P, HKV, D), W.BF16_NAN, np.uint16)
    v16 = k16.copy()
    q4 = empty_q4_pools(pages)
    used = 0
    for b, L in enumerate(lens):
        n = W.pages_for(int(L))
        bt[b, :n] = perm[used:used + n]
        used += n
        if L:
            kr, vr = rows_fn(rng, int(L)), rows_fn(rng, int(L))
            k16, v16 = oracle.fill_kv(k16, v16, kr, vr, bt[b], 0)
            q4 = kq.fill_kv_q8(*q4, kr, vr, bt[b], 0, nbits=4)
    return k16, v16, q4, bt


def pin_q4_lossless_rows_match_bf16_attention(kq):
    rng = np.random.default_rng(715)
    lens = np.array([1, 16, 33, 0, 70], np.int32)
    k16, v16, (kc, vc, sc), bt = _fill_both_q4(kq, rng, lens, 24, exact_grid_rows_q4)
    q = W.random_q(rng, len(lens))
    want = oracle.decode_attention(q, k16, v16, bt, lens, W.SCALE)
    got = kq.decode_attention_q8(q, kc, vc, sc, bt, lens, W.SCALE, nbits=4)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    for b, L in enumerate(lens):
        K = kq.gather_sequence_q8(kc, sc, 0, bt[b], int(L), nbits=4)
        V = kq.gather_sequence_q8(vc, sc, 1, bt[b], int(L), nbits=4)
        assert np.array_equal(K, oracle.gather_sequence(k16, bt[b], int(L)))
        assert np.array_equal(V, oracle.gather_sequence(v16, bt[b], int(L)))


def pin_q4_error_within_bound(kq):
    rng = np.random.default_rng(716)
    lens = np.array([5, 200, 64], np.int32)
    k16, v16, (kc, vc, sc), bt = _fill_both_q4(kq, rng, lens, 24, W.random_rows)
    q = W.random_q(rng, len(lens))
    ref = oracle.decode_attention(q, k16, v16, bt, lens, W.SCALE)
    got = kq.decode_attention_q8(q, kc, vc, sc, bt, lens, W.SCALE, nbits=4)
    qf = oracle.bf16_bits_to_f64(q)
    worst, worst_bound = 0.0, 0.0
    for b, L in enumerate(lens):
        K, V = oracle.gather_sequence(k16, bt[b], int(L)), oracle.gather_sequence(v16, bt[b], int(L))
        Kh = kq.gather_sequence_q8(kc, sc, 0, bt[b], int(L), nbits=4)
        Vh = kq.gather_sequence_q8(vc, sc, 1, bt[b], int(L), nbits=4)
        for h in range(HQ):
            g = h // (HQ // HKV)
            bound = kq.quantisation_error_bound(qf[b, h], K[:, g], Kh[:, g], V[:, g], Vh[:, g], W.SCALE)
            err = np.abs(got[b, h] - ref[b, h])
            assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (b, h)
            worst = max(worst, float(np.max(err)))
            worst_bound = max(worst_bound, float(np.max(bound)))
    assert worst > 0
    assert worst_bound < 3.0                                 # the bound says something


ALL_Q4_PINS = [
    pin_q4_golden_rows,
    pin_q4_brute_force_nearest_code,
    pin_q4_invariants,
    pin_q4_packing_round_trip,
    pin_q4_append_touches_one_slot,
    pin_q4_fill_equals_appends,
    pin_q4_lossless_rows_match_bf16_attention,
    pin_q4_error_within_bound,
]
