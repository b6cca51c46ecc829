"""Pins for the RoPE step of the oracle (closed forms and invariants).

Each pin takes the oracle's rope module (or a copy with a planted mistake).
Expected values come from the rotation's definition worked by hand, from
float64 rotations, and from the BF16 rounding rule applied to chosen values.
"""

from __future__ import annotations

import numpy as np

import workloads as W
from oracle_pins import exact_bf16, lib_decode

D = W.HEAD_DIM
H = D // 2


def _tables(rows):
    cos = np.array([r[0] for r in rows], dtype=np.float32)
    sin = np.array([r[1] for r in rows], dtype=np.float32)
    return cos, sin


def pin_rope_identity_at_zero_angle(rope):
    rng = np.random.default_rng(301)
    x = W.random_q(rng, 1)[0]                                  # [32][64] bf16 bits
    got = rope.f32_to_bf16_bits_rne(rope.rope_rotate_f32(x, np.ones(H), np.zeros(H)))
    assert np.array_equal(got, x)


def pin_rope_quarter_turn_pairs_rotate_half(rope):
    """cos 0, sin 1 maps (x_i, x_{i+32}) to (-x_{i+32}, x_i) exactly (rotate-half pairs)."""
    vals = np.arange(1, D + 1, dtype=np.float64)               # exact in BF16
    x = exact_bf16(vals[None, :])
    got = rope.rope_rotate_f32(x, np.zeros(H), np.ones(H))[0]
    want = np.concatenate([-vals[H:], vals[:H]])
    assert np.array_equal(got.astype(np.float64), want)


def pin_rope_matches_float64_rotation(rope):
    rng = np.random.default_rng(302)
    cos, sin = W.rope_table(300)
    x = W.random_rows(rng, 300)                                # [300][8][64]
    for pos in (0, 1, 17, 299):
        got = rope.rope_rotate_f32(x[pos], cos[pos], sin[pos]).astype(np.float64)
        xf = lib_decode(x[pos]).numpy()
        c, s = cos[pos].astype(np.float64), sin[pos].astype(np.float64)
        want = np.concatenate([xf[:, :H] * c - xf[:, H:] * s, xf[:, H:] * c + xf[:, :H] * s], 1)
        np.testing.assert_allclose(got, want, rtol=0, atol=4e-6 * np.abs(xf).max())
        # a rotation keeps the length of every pair
        n_in = xf[:, :H] ** 2 + xf[:, H:] ** 2
        n_out = got[:, :H] ** 2 + got[:, H:] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=2e-6, atol=1e-12)


def pin_rope_relative_position(rope):
    """q.k after rotating by positions (m, n) equals that after (m + d, n + d)."""
    rng = np.random.default_rng(303)
    cos, sin = W.rope_table(2048)
    q = W.random_q(rng, 1)[0, :1]
    k = W.random_rows(rng, 1)[0, :1]
    def dot(m, n):
        a = rope.rope_rotate_f32(q, cos[m], sin[m]).astype(np.float64)
        b = rope.rope_rotate_f32(k, cos[n], sin[n]).astype(np.float64)
        return float((a * b).sum())
    for m, n, d in ((5, 3, 100), (1000, 20, 1000), (0, 7, 2000)):
        assert abs(dot(m, n) - dot(m + d, n + d)) < 2e-4 * (1 + abs(dot(m, n)))


def pin_rope_rounds_to_nearest_even(rope):
    # halfway cases: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6; just above half -> up;
    # the carry out of the fraction into the exponent; negatives mirror positives
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,
                  2 - 2.0 ** -9, -(1 + 3 * 2.0 ** -8), 3.0], dtype=np.float32)
    assert list(rope.f32_to_bf16_bits_rne(x)) == [0x3F80, 0x3F82, 0x3F81, 0x4000, 0xBF82, 0x4040]


def pin_rope_new_token_uses_position_L_minus_1(rope):
    """Only the row of position L-1 turns a quarter; every other position is the identity."""
    lens = np.array([1, 5, 16, 17, 0], dtype=np.int32)
    rng = np.random.default_rng(304)
    q = W.random_q(rng, len(lens))
    k = W.random_rows(rng, len(lens))
    for b, L in enumerate(lens):
        if L == 0:
            continue
        cos = np.ones((32, H), np.float32)
        sin = np.zeros((32, H), np.float32)
        cos[L - 1], sin[L - 1] = 0.0, 1.0
        q_rot, k_rot = rope.rope_new_token(q, k, lens, cos, sin)
        qf = lib_decode(q[b]).numpy()
        kf = lib_decode(k[b]).numpy()
        assert np.array_equal(lib_decode(q_rot[b]).numpy(),
                              np.concatenate([-qf[:, H:], qf[:, :H]], 1))
        assert np.array_equal(lib_decode(k_rot[b]).numpy(),
                              np.concatenate([-kf[:, H:], kf[:, :H]], 1))
    q_rot, k_rot = rope.rope_new_token(q, k, lens, np.ones((32, H), np.float32),
                                       np.zeros((32, H), np.float32))
    assert np.array_equal(q_rot[4], q[4]) and np.array_equal(k_rot[4], k[4])


ALL_ROPE_PINS = [
    pin_rope_identity_at_zero_angle,
    pin_rope_quarter_turn_pairs_rotate_half,
    pin_rope_matches_float64_rotation,
    pin_rope_relative_position,
    pin_rope_rounds_to_nearest_even,
    pin_rope_new_token_uses_position_L_minus_1,
]
