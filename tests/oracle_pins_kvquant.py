"""Pins for the INT8 K/V page oracle (hand-worked values, brute force, exact cases, a bound).

Each pin takes the oracle's kvquant module (or a copy with a planted
mistake).  What fixes the expected values:

* the hand-worked rows of ``golden/int8_quant_examples.json`` (the pages'
  symmetric quantiser with power-of-two scales, ties to even);
* brute force: every code is the integer nearest the FP32 quotient, found by
  trying all 256 codes with exact rational comparisons;
* invariants of the quantiser (the largest magnitude maps to +-127, the
  reconstruction error is at most half a scale);
* lossless cases: rows built as integer codes times a power of two
  quantise without error, so attention over the INT8 pages must equal the
  BF16 oracle's attention on the same values to float64 rounding;
* the analytic bound on how far quantisation moves the attention output
  (derived in the oracle's docstring), checked against the BF16 oracle on
  random data.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads as W

HKV, D, P, HQ = W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE, W.NUM_Q_HEADS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_quant_examples.json")


def _bits(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def empty_q8_pools(pages):
    return (np.zeros((pages, HKV, P, D), np.int8), np.zeros((pages, HKV, P, D), np.int8),
            np.zeros((pages, HKV, 2, P), np.float32))


def exact_grid_rows(rng, n):
    """``[n][Hkv][D]`` BF16 rows that INT8 holds exactly: codes in [-127, 127]
    (one of them +-127) times 2^e, e in -6..0, per (token, head) row."""
    codes = rng.integers(-127, 128, size=(n, HKV, D))
    pick = rng.integers(0, D, size=(n, HKV))
    sign = rng.choice([-1, 1], size=(n, HKV))
    np.put_along_axis(codes, pick[..., None], (127 * sign)[..., None], axis=-1)
    e = rng.integers(-6, 1, size=(n, HKV, 1)).astype(np.float64)
    vals = codes * np.exp2(e)
    return _bits(vals)


# ---------------------------------------------------------------------------
# The quantiser
# ---------------------------------------------------------------------------
def pin_q8_golden_rows(kq):
    g = json.load(open(GOLDEN))
    rows = np.array([r["values"] for r in g["rows"]], dtype=np.float32)
    codes, scale = kq.quantize_rows(_bits(rows))
    assert np.array_equal(scale.astype(np.float64), [r["scale"] for r in g["rows"]])
    assert np.array_equal(codes.astype(np.int64), np.array([r["codes"] for r in g["rows"]]))
    assert codes.dtype == np.int8 and scale.dtype == np.float32


def pin_q8_brute_force_nearest_code(kq):
    rng = np.random.default_rng(611)
    x = W.random_rows(rng, 3)[:, :, :16]                    # 24 rows of 16 values
    codes, scale = kq.quantize_rows(x)
    xf = oracle.bf16_bits_to_f64(x)
    for idx in np.ndindex(*x.shape[:-1]):
        s = np.float32(scale[idx])
        # the scale: the FP32 number nearest max|x| / 127
        amax = Fraction(float(np.max(np.abs(xf[idx]))))
        assert abs(Fraction(float(s)) - amax / 127) <= abs(Fraction(float(np.nextafter(s, np.inf))) - amax / 127)
        assert abs(Fraction(float(s)) - amax / 127) <= abs(Fraction(float(np.nextafter(s, -np.inf))) - amax / 127)
        for j in range(x.shape[-1]):
            r = Fraction(float(np.float32(np.float32(xf[idx][j]) / s)))   # FP32 quotient
            best = min(range(-128, 128), key=lambda c: (abs(r - c), c % 2))
            assert int(codes[idx][j]) == best, (idx, j)


def pin_q8_invariants(kq):
    rng = np.random.default_rng(612)
    x = W.random_rows(rng, 64)
    x[3, 5] = 0                                             # one zero row
    codes, scale = kq.quantize_rows(x)
    xf = oracle.bf16_bits_to_f64(x)
    amax = np.max(np.abs(xf), axis=-1)
    live = amax > 0
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)
    assert np.array_equal(np.max(np.abs(codes.astype(np.int64)), axis=-1)[live], np.full(live.sum(), 127))
    s = scale.astype(np.float64)
    assert np.all(np.abs(127 * s - amax) <= amax * 2.0 ** -23)
    err = np.abs(xf - codes * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 2.0 ** -16))
    assert scale[3, 5] == 0 and not np.any(codes[3, 5])


def pin_q8_dequantize_exact(kq):
    codes = np.array([[-128, -127, -1, 0, 1, 127]], dtype=np.int8)
    scale = np.array([np.float32(3.0e-3)], dtype=np.float32)
    got = kq.dequantize(codes, scale)
    want = np.array([[c * float(scale[0]) for c in (-128, -127, -1, 0, 1, 127)]])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# Pages
# ---------------------------------------------------------------------------
def pin_q8_append_touches_one_slot(kq):
    rng = np.random.default_rng(613)
    pages = 12
    kc, vc, sc = empty_q8_pools(pages)
    kc[:] = rng.integers(-128, 128, kc.shape)
    vc[:] = rng.integers(-128, 128, vc.shape)
    sc[:] = rng.random(sc.shape, dtype=np.float32)
    bt = np.array([[7, 2, 9], [4, 0, 1], [3, 5, 6]], np.int32)
    lens = np.array([17, 0, 48], np.int32)                  # slot 0 of page 2; idle; slot 15 of page 6
    kn, vn = W.random_rows(rng, 3), W.random_rows(rng, 3)
    k2, v2, s2 = kq.append_kv_q8(kc, vc, sc, kn, vn, bt, lens)
    changed = {(int(p), int(t)) for p, t in zip(*np.nonzero(np.any(k2 != kc, axis=(1, 3))))}
    assert changed <= {(2, 0), (6, 15)}
    for b, (page, slot) in ((0, (2, 0)), (2, (6, 15))):
        ck, skk = kq.quantize_rows(kn[b])
        cv, svv = kq.quantize_rows(vn[b])
        assert np.array_equal(k2[page, :, slot], ck) and np.array_equal(v2[page, :, slot], cv)
        assert np.array_equal(s2[page, :, 0, slot], skk) and np.array_equal(s2[page, :, 1, slot], svv)
    mask = np.ones(sc.shape, bool)
    mask[2, :, :, 0] = False
    mask[6, :, :, 15] = False
    assert np.array_equal(s2[mask], sc[mask])
    vmask = np.ones((pages, P), bool)
    vmask[2, 0] = vmask[6, 15] = False
    v2t, vct = np.swapaxes(v2, 1, 2), np.swapaxes(vc, 1, 2)          # [page][slot][head][dim]
    assert np.array_equal(v2t[vmask], vct[vmask])


def pin_q8_fill_equals_appends(kq):
    rng = np.random.default_rng(614)
    pages, T, start = 10, 37, 5
    kc, vc, sc = empty_q8_pools(pages)
    row = rng.permutation(pages)[: W.pages_for(start + T)].astype(np.int32)
    kr, vr = W.random_rows(rng, T), W.random_rows(rng, T)
    f = kq.fill_kv_q8(kc, vc, sc, kr, vr, row, start)
    a = (kc, vc, sc)
    for j in range(T):
        a = kq.append_kv_q8(*a, kr[j:j + 1], vr[j:j + 1], row[None, :], np.array([start + j + 1], np.int32))
    for x, y in zip(f, a):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# Attention over the pages
# ---------------------------------------------------------------------------
def _fill_both(kq, rng, lens, pages, rows_fn):
    """BF16 pools and INT8 pools holding the same rows (placed at random)."""
    B = len(lens)
    mb = max(W.pages_for(int(L)) for L in lens) + 1
    perm = rng.permutation(pages)
    bt = np.full((B, mb), -1, np.int32)
    k16 = np.full((pages, P, HKV, D), W.BF16_NAN, np.uint16)
    v16 = k16.copy()
    q8 = empty_q8_pools(pages)
    used = 0
    for b, L in enumerate(lens):
        n = W.pages_for(int(L))
        bt[b, :n] = perm[used:used + n]
        used += n
        if L:
            kr, vr = rows_fn(rng, int(L)), rows_fn(rng, int(L))
            k16, v16 = oracle.fill_kv(k16, v16, kr, vr, bt[b], 0)
            q8 = kq.fill_kv_q8(*q8, kr, vr, bt[b], 0)
    return k16, v16, q8, bt


def pin_q8_lossless_rows_match_bf16_attention(kq):
    rng = np.random.default_rng(615)
    lens = np.array([1, 16, 33, 0, 70], np.int32)
    k16, v16, (kc, vc, sc), bt = _fill_both(kq, rng, lens, 24, exact_grid_rows)
    q = W.random_q(rng, len(lens))
    want = oracle.decode_attention(q, k16, v16, bt, lens, W.SCALE)
    got = kq.decode_attention_q8(q, kc, vc, sc, bt, lens, W.SCALE)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # and the lossless rows really did keep every value
    for b, L in enumerate(lens):
        K = kq.gather_sequence_q8(kc, sc, 0, bt[b], int(L))
        V = kq.gather_sequence_q8(vc, sc, 1, bt[b], int(L))
        assert np.array_equal(K, oracle.gather_sequence(k16, bt[b], int(L)))
        assert np.array_equal(V, oracle.gather_sequence(v16, bt[b], int(L)))


def pin_q8_error_within_bound(kq):
    rng = np.random.default_rng(616)
    lens = np.array([5, 200, 64], np.int32)
    k16, v16, (kc, vc, sc), bt = _fill_both(kq, rng, lens, 24, W.random_rows)
    q = W.random_q(rng, len(lens))
    ref = oracle.decode_attention(q, k16, v16, bt, lens, W.SCALE)
    got = kq.decode_attention_q8(q, kc, vc, sc, bt, lens, W.SCALE)
    qf = oracle.bf16_bits_to_f64(q)
    worst = 0.0
    for b, L in enumerate(lens):
        K, V = oracle.gather_sequence(k16, bt[b], int(L)), oracle.gather_sequence(v16, bt[b], int(L))
        Kh = kq.gather_sequence_q8(kc, sc, 0, bt[b], int(L))
        Vh = kq.gather_sequence_q8(vc, sc, 1, bt[b], int(L))
        for h in range(HQ):
            g = h // (HQ // HKV)
            bound = kq.quantisation_error_bound(qf[b, h], K[:, g], Kh[:, g], V[:, g], Vh[:, g], W.SCALE)
            err = np.abs(got[b, h] - ref[b, h])
            assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (b, h)
            assert float(np.max(bound)) < 0.15               # the bound says something
            worst = max(worst, float(np.max(err)))
    assert worst > 0                                        # quantisation did change the output


ALL_KVQUANT_PINS = [
    pin_q8_golden_rows,
    pin_q8_brute_force_nearest_code,
    pin_q8_invariants,
    pin_q8_dequantize_exact,
    pin_q8_append_touches_one_slot,
    pin_q8_fill_equals_appends,
    pin_q8_lossless_rows_match_bf16_attention,
    pin_q8_error_within_bound,
]
