"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an oracle module (the real one, or a copy with a
planted mistake) and raises ``AssertionError`` when the oracle disagrees with a
closed form, an invariant or a library routine.  Expected values never come
from the oracle under test: BF16 bits are decoded with torch's own bfloat16
type, attention is recomputed with ``torch.nn.functional.
scaled_dot_product_attention`` in float64, and means, sums and permutations
are taken on the logical arrays before they are paged.

Reading shared with the oracle and restated here: query head ``h`` reads KV
head ``h // 4`` (32 query heads over 8 KV heads).
"""

from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W

HQ, HKV, D, P = W.NUM_Q_HEADS, W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE
G = HQ // HKV
SCALE = W.SCALE


def lib_decode(bits) -> torch.Tensor:
    """BF16 bits -> float64 through torch's bfloat16 dtype (independent code)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64)


def exact_bf16(values) -> np.ndarray:
    """BF16 bits of values that BF16 represents exactly (asserted)."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float64))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t), "value not exact in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


def sdpa_reference(q_bits, k_rows, v_rows, scale=SCALE) -> np.ndarray:
    """[B][HQ][D] float64 attention of each sequence's logical rows via torch."""
    out = []
    for b in range(len(k_rows)):
        q = lib_decode(q_bits[b]).unsqueeze(1)                    # [HQ][1][D]
        if k_rows[b].shape[0] == 0:
            out.append(np.zeros((HQ, D)))
            continue
        K = lib_decode(k_rows[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [HQ][L][D]
        V = lib_decode(v_rows[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, K.contiguous(), V.contiguous(), scale=scale)
        out.append(o.squeeze(1).numpy())
    return np.stack(out)


def _run(ora, batch, **kw):
    return ora.decode_attention(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                                batch.seq_lens, batch.scale, **kw)


def _rand_case(seed, lens, q_sigma=1.0):
    rng = np.random.default_rng(seed)
    q = W.random_q(rng, len(lens), q_sigma)
    k = [W.random_rows(rng, L) for L in lens]
    v = [W.random_rows(rng, L) for L in lens]
    return q, k, v


def _pool_pages(lens, slack=7):
    return sum(W.pages_for(L) for L in lens) + slack


# --------------------------------------------------------------------------
def pin_seq_len_one(ora):
    """L = 1: the only weight is 1, so every head returns its KV head's V row exactly."""
    lens = [1, 1, 1]
    q, k, v = _rand_case(101, lens)
    batch = W.pack_logical(q, k, v, _pool_pages(lens), seed=7)
    out = _run(ora, batch)
    for b in range(len(lens)):
        V0 = lib_decode(v[b][0]).numpy()                      # [HKV][D]
        for h in range(HQ):
            assert np.array_equal(out[b, h], V0[h // G]), (b, h)


def pin_identical_values(ora):
    """All V rows equal to r: the convex combination returns r."""
    lens = [5, 16, 37]
    rng = np.random.default_rng(102)
    q = W.random_q(rng, len(lens))
    k = [W.random_rows(rng, L) for L in lens]
    v = []
    rows = []
    for L in lens:
        r = W.random_rows(rng, 1)
        rows.append(lib_decode(r[0]).numpy())
        v.append(np.repeat(r, L, axis=0))
    out = _run(ora, W.pack_logical(q, k, v, _pool_pages(lens), seed=8))
    for b in range(len(lens)):
        for h in range(HQ):
            np.testing.assert_allclose(out[b, h], rows[b][h // G], rtol=0, atol=1e-13)


def pin_equal_scores_mean(ora):
    """q = 0 (or all K rows equal): every score ties, the output is the mean of V[0..L).

    Lengths end mid-page, on a page boundary and one past it, so the tail
    slots (poisoned with NaN) must not be read.
    """
    lens = [1, 5, 15, 16, 17, 37, 100]
    rng = np.random.default_rng(103)
    k = [W.random_rows(rng, L) for L in lens]
    v = [W.random_rows(rng, L) for L in lens]
    q0 = np.zeros((len(lens), HQ, D), dtype=np.uint16)
    out = _run(ora, W.pack_logical(q0, k, v, _pool_pages(lens), seed=9))
    for b in range(len(lens)):
        mean = lib_decode(v[b]).mean(dim=0).numpy()              # [HKV][D]
        for h in range(HQ):
            np.testing.assert_allclose(out[b, h], mean[h // G], rtol=0, atol=1e-13)
    # same with a random query and identical K rows
    qr = W.random_q(rng, len(lens))
    k_same = [np.repeat(W.random_rows(rng, 1), L, axis=0) for L in lens]
    out = _run(ora, W.pack_logical(qr, k_same, v, _pool_pages(lens), seed=10))
    for b in range(len(lens)):
        mean = lib_decode(v[b]).mean(dim=0).numpy()
        for h in range(HQ):
            np.testing.assert_allclose(out[b, h], mean[h // G], rtol=0, atol=1e-13)


def pin_weights_sum_to_one(ora):
    """Softmax weights: one per attended token, non-negative, summing to 1."""
    lens = [1, 7, 33]
    q, k, v = _rand_case(104, lens)
    out, weights = _run(ora, W.pack_logical(q, k, v, _pool_pages(lens), seed=11),
                        return_weights=True)
    for b, L in enumerate(lens):
        for h in range(HQ):
            w = np.asarray(weights[(b, h)])
            assert w.shape == (L,)
            assert np.all(w >= 0)
            assert abs(w.sum() - 1.0) < 1e-14


def pin_page_shuffle_bitwise(ora):
    """Moving physical pages (and rewriting the block table) changes nothing, bit for bit."""
    lens = [3, 16, 17, 64, 129]
    q, k, v = _rand_case(105, lens)
    pages = _pool_pages(lens, slack=40)
    a = _run(ora, W.pack_logical(q, k, v, pages, seed=12))
    b = _run(ora, W.pack_logical(q, k, v, pages, seed=13))
    c = _run(ora, W.pack_logical(q, k, v, pages, seed=0, placement="identity"))
    assert np.array_equal(a, b) and np.array_equal(a, c)


def pin_token_permutation(ora):
    """Single-query attention ignores token order (K and V rows permuted together)."""
    lens = [9, 40]
    q, k, v = _rand_case(106, lens)
    rng = np.random.default_rng(0)
    perm = [rng.permutation(L) for L in lens]
    k2 = [k[i][perm[i]] for i in range(len(lens))]
    v2 = [v[i][perm[i]] for i in range(len(lens))]
    pages = _pool_pages(lens)
    a = _run(ora, W.pack_logical(q, k, v, pages, seed=14))
    b = _run(ora, W.pack_logical(q, k2, v2, pages, seed=14))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_value_shift_and_linearity(ora):
    """o(V + c) = o(V) + c and o(V1 + V2) = o(V1) + o(V2) (weights do not depend on V).

    V entries are small integers so the shifted and summed rows stay exact in BF16.
    """
    lens = [4, 21]
    rng = np.random.default_rng(107)
    q = W.random_q(rng, len(lens))
    k = [W.random_rows(rng, L) for L in lens]
    v1 = [rng.integers(-8, 9, size=(L, HKV, D)).astype(np.float64) for L in lens]
    v2 = [rng.integers(-8, 9, size=(L, HKV, D)).astype(np.float64) for L in lens]
    pages = _pool_pages(lens)

    def o(vals):
        return _run(ora, W.pack_logical(q, k, [exact_bf16(x) for x in vals], pages, seed=15))

    base, other = o(v1), o(v2)
    shifted = o([x + 16.0 for x in v1])
    summed = o([x + y for x, y in zip(v1, v2)])
    np.testing.assert_allclose(shifted, base + 16.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(summed, base + other, rtol=0, atol=1e-12)


def pin_library_attention(ora):
    """Brute force against torch's scaled_dot_product_attention in float64."""
    lens = [1, 2, 3, 15, 16, 17, 37, 100, 300]
    q, k, v = _rand_case(108, lens)
    out = _run(ora, W.pack_logical(q, k, v, _pool_pages(lens), seed=16))
    ref = sdpa_reference(q, k, v)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_hand_example_two_tokens(ora):
    """A case worked by hand: scores 1 and 0 give weights sigmoid(1) and sigmoid(-1).

    Every query head has q[0] = 8 and zeros elsewhere; token 0's keys have
    k[0] = 1, token 1's keys are zero; so with scale 1/8 the scores are 1 and
    0.  V rows are small integers.  Expected output, by hand:
    o = s(1) * v0 + s(-1) * v1 with s(x) = 1 / (1 + exp(-x)).
    """
    q = np.zeros((1, HQ, D)); q[0, :, 0] = 8.0
    k = np.zeros((2, HKV, D)); k[0, :, 0] = 1.0
    rng = np.random.default_rng(109)
    v = rng.integers(-5, 6, size=(2, HKV, D)).astype(np.float64)
    batch = W.pack_logical(exact_bf16(q), [exact_bf16(k)], [exact_bf16(v)], 4, seed=17)
    out = _run(ora, batch)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    s0 = 1.0 / (1.0 + math.exp(1.0))
    for h in range(HQ):
        np.testing.assert_allclose(out[0, h], s1 * v[0, h // G] + s0 * v[1, h // G],
                                   rtol=0, atol=1e-14)


def pin_gqa_one_hot(ora):
    """Only KV head g* carries non-zero V: only query heads 4g*..4g*+3 answer non-zero.

    A second case gives the four query heads of a group identical rows; their
    outputs must then be identical.
    """
    lens = [6, 19]
    rng = np.random.default_rng(110)
    q = W.random_q(rng, len(lens))
    k = [W.random_rows(rng, L) for L in lens]
    pages = _pool_pages(lens)
    for gstar in range(HKV):
        v = []
        for L in lens:
            vals = np.zeros((L, HKV, D))
            vals[:, gstar, :] = rng.integers(1, 4, size=(L, D))
            v.append(exact_bf16(vals))
        out = _run(ora, W.pack_logical(q, k, v, pages, seed=18))
        for h in range(HQ):
            nonzero = np.any(out[:, h] != 0)
            assert nonzero == (h // G == gstar), (gstar, h)
    q_same = q.copy()
    for g in range(HKV):
        q_same[:, G * g:G * g + G] = q[:, G * g:G * g + 1]
    v = [W.random_rows(rng, L) for L in lens]
    out = _run(ora, W.pack_logical(q_same, k, v, pages, seed=19))
    for g in range(HKV):
        for j in range(1, G):
            assert np.array_equal(out[:, G * g + j], out[:, G * g])


def pin_split_merge(ora):
    """Attention over a partition of [0, L), merged by log-sum-exp, equals the whole.

    For parts s with outputs o_s and log-sum-exp values z_s, the whole has
    z = log(sum_s exp(z_s)) and o = sum_s exp(z_s - z) * o_s.
    """
    L = 70
    q, k, v = _rand_case(111, [L])
    cuts = [0, 16, 17, 48, 70]
    whole, lse_whole = _run(ora, W.pack_logical(q, k, v, 12, seed=20), return_lse=True)
    parts, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, z = _run(ora, W.pack_logical(q, [k[0][a:b]], [v[0][a:b]], 12, seed=21),
                    return_lse=True)
        parts.append(o[0]); lses.append(z[0])
    lses = np.stack(lses)                                  # [S][HQ]
    top = lses.max(axis=0)
    z = top + np.log(np.exp(lses - top).sum(axis=0))
    merged = sum(np.exp(lses[s] - z)[:, None] * parts[s] for s in range(len(parts)))
    np.testing.assert_allclose(merged, whole[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(z, lse_whole[0], rtol=0, atol=1e-12)


def pin_idle_slot(ora):
    """seq_len 0 marks an idle batch slot: its output row is zero, the others are unaffected."""
    lens = [0, 9, 0]
    q, k, v = _rand_case(112, lens)
    out = _run(ora, W.pack_logical(q, k, v, 4, seed=22))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    np.testing.assert_allclose(out[1], sdpa_reference(q[1:2], k[1:2], v[1:2])[0],
                               rtol=0, atol=1e-12)


def pin_append_positions(ora):
    """Appending token L-1 to a pool holding tokens 0..L-2 gives, byte for byte, the
    pool the generator builds directly with tokens 0..L-1 (same placement).

    Lengths cover the first slot of a page, its last slot and the last slot of
    a full 2,048-token context; an idle slot (L = 0) writes nothing.
    """
    lens = [1, 2, 15, 16, 17, 32, 33, 2047, 2048, 0]
    q, k, v = _rand_case(113, lens)
    pages = _pool_pages(lens, slack=5)
    pre = W.pack_logical(q, [x[:max(L - 1, 0)] for x, L in zip(k, lens)],
                         [x[:max(L - 1, 0)] for x, L in zip(v, lens)], pages, seed=23,
                         capacity=lens)
    post = W.pack_logical(q, k, v, pages, seed=23, capacity=lens)
    assert np.array_equal(pre.block_tables, post.block_tables)
    k_new = np.stack([x[L - 1] if L else np.zeros((HKV, D), np.uint16) for x, L in zip(k, lens)])
    v_new = np.stack([x[L - 1] if L else np.zeros((HKV, D), np.uint16) for x, L in zip(v, lens)])
    k_out, v_out = ora.append_kv(pre.k_pool, pre.v_pool, k_new, v_new,
                                 pre.block_tables, pre.seq_lens)
    assert np.array_equal(k_out, post.k_pool)
    assert np.array_equal(v_out, post.v_pool)
    # inputs untouched
    assert not np.array_equal(pre.k_pool, post.k_pool)


def pin_fill_positions(ora):
    """Filling tokens start .. start+T-1 of each sequence into a pool that holds
    tokens 0 .. start-1 gives, byte for byte, the pool the generator builds
    directly with tokens 0 .. start+T-1 (same placement).

    Spans start at a page's first slot, end on its last, cross page boundaries,
    fill one token, and reach the last slot of a 2,048-token context.
    """
    spans = [(0, 37), (15, 2), (16, 16), (0, 1), (2000, 48), (33, 300), (7, 9)]
    lens = [s + t for s, t in spans]
    q, k, v = _rand_case(114, lens)
    pages = _pool_pages(lens, slack=5)
    pre = W.pack_logical(q, [x[:s] for x, (s, _) in zip(k, spans)],
                         [x[:s] for x, (s, _) in zip(v, spans)], pages, seed=24, capacity=lens)
    post = W.pack_logical(q, k, v, pages, seed=24, capacity=lens)
    assert np.array_equal(pre.block_tables, post.block_tables)
    k_out, v_out = pre.k_pool, pre.v_pool
    for b, (s, t) in enumerate(spans):
        k_out, v_out = ora.fill_kv(k_out, v_out, k[b][s:s + t], v[b][s:s + t],
                                   pre.block_tables[b], s)
    assert np.array_equal(k_out, post.k_pool)
    assert np.array_equal(v_out, post.v_pool)
    # inputs untouched
    assert not np.array_equal(pre.k_pool, post.k_pool)


ALL_PINS = [
    pin_seq_len_one,
    pin_identical_values,
    pin_equal_scores_mean,
    pin_weights_sum_to_one,
    pin_page_shuffle_bitwise,
    pin_token_permutation,
    pin_value_shift_and_linearity,
    pin_library_attention,
    pin_hand_example_two_tokens,
    pin_gqa_one_hot,
    pin_split_merge,
    pin_idle_slot,
    pin_append_positions,
    pin_fill_positions,
]
