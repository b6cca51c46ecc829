"""The bit identities the INT4 decode kernel widens its codes with, on the CPU.

The kernel never converts an INT4 code: it masks a nibble u = code + 8 into a
BF16 bit pattern whose value is u plus a fixed offset, multiplies exactly on
the matrix cores and takes the offset back out (include/pa_decode_q4.h; the
INT4 cache is the lower-precision cache of the llm-inference article, section
5.1, quantised with its section 3.4 quantiser at 4 bits).  These tests pin the
identities themselves against the oracle's unpacking of the same bytes:

* 0x4300 | u is 128 + u, so a first nibble (bits 0..3 of a 16-bit unit) reads
  code + 136 with no shift;
* 0x4180 | (u << 3) is 16 + u, so nibbles 1..3, shifted down to bits 3..6,
  read code + 24;
* one 64-bit shift of two packed words serves both: the bits it carries from
  the high word into the low one fall outside the mask;
* the pair order of a word is dims 0 4 1 5 2 6 3 7;
* taking the offsets out with the weights the products carry (the BF16 weight
  plus its BF16 remainder) leaves no multiple of the offset behind.
"""

from __future__ import annotations

import numpy as np

from oracle import kvquant


def bf16(bits):
    """BF16 bit patterns (uint16 or the halves of uint32 words) -> float64."""
    b = np.asarray(bits, np.uint32) & 0xFFFF
    return (b << 16).view(np.float32).astype(np.float64)


def test_every_nibble_widens_to_its_offset_value():
    u = np.arange(16, dtype=np.uint32)
    assert np.array_equal(bf16(0x4300 | u), 128.0 + u)
    assert np.array_equal(bf16(0x4180 | (u << 3)), 16.0 + u)
    # code = u - 8: the offsets are 136 and 24
    assert np.array_equal(bf16(0x4300 | u) - 136.0, u.astype(np.float64) - 8)
    assert np.array_equal(bf16(0x4180 | (u << 3)) - 24.0, u.astype(np.float64) - 8)


def widen_pair(w_lo, w_hi, e):
    """Nibble pair e of two packed 32-bit words -> two words of two BF16 each,
    as the kernel computes it (one 64-bit shift, one mask-and-or per word)."""
    w = (np.uint64(w_hi) << np.uint64(32)) | np.uint64(w_lo)
    if e == 0:
        mask, bias, f = 0x000F000F, 0x43004300, w
    else:
        mask, bias, f = 0x00780078, 0x41804180, w >> np.uint64(4 * e - 3)
    o0 = (int(f) & 0xFFFFFFFF & mask) | bias
    o1 = ((int(f) >> 32) & mask) | bias
    return o0, o1


def test_packed_words_widen_to_the_oracle_codes_in_pair_order():
    rng = np.random.default_rng(4242)
    for _ in range(200):
        codes = rng.integers(-8, 8, size=16)          # dims 16G .. 16G+15 of one token
        packed = kvquant.pack_q4(codes)                # 8 bytes
        w0, w1 = (int(x) for x in packed.view(np.uint32))
        got0, got1 = [], []
        for e in range(4):
            o0, o1 = widen_pair(w0, w1, e)
            off = 136.0 if e == 0 else 24.0
            got0 += [bf16(o0) - off, bf16(o0 >> 16) - off]
            got1 += [bf16(o1) - off, bf16(o1 >> 16) - off]
        order = [0, 4, 1, 5, 2, 6, 3, 7]
        assert np.array_equal(np.array(got0).ravel(), codes[:8][order].astype(np.float64))
        assert np.array_equal(np.array(got1).ravel(), codes[8:][order].astype(np.float64))


def test_offsets_leave_with_the_carried_weights():
    """acc = sum (w_hi + w_lo)(code + b) and wsum = sum (w_hi + w_lo): acc - b wsum is
    sum (w_hi + w_lo) code up to FP32 accumulation, while wsum = sum w would leave
    b * sum (w - w_hi - w_lo) behind."""
    rng = np.random.default_rng(7)

    def to_bf16(x):
        x = np.asarray(x, np.float32)
        b = x.view(np.uint32)
        r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)   # round to nearest even
        return (r << 16).view(np.float32)

    w = rng.uniform(0.0, 0.5, size=16).astype(np.float32)
    hi = to_bf16(w)
    lo = to_bf16(w - hi)
    carried = hi.astype(np.float64) + lo.astype(np.float64)
    codes = rng.integers(-8, 8, size=16).astype(np.float64)
    for b in (24.0, 136.0):
        acc = np.sum(carried * (codes + b))
        exact = np.sum(carried * codes)
        assert abs((acc - b * carried.sum()) - exact) < 1e-12
        leftover = abs((acc - b * w.astype(np.float64).sum()) - exact)
        assert np.isclose(leftover, abs(b * (w.astype(np.float64) - carried).sum()), rtol=1e-9, atol=0)
