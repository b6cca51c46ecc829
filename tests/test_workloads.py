"""The seeded input generator: reproducible, poisoned, and shaped as the workloads say."""

import numpy as np

import workloads as W


def test_seed_reproduces_every_byte():
    a = W.make_workload(2)
    b = W.make_workload(2)
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool),
                 (a.block_tables, b.block_tables), (a.seq_lens, b.seq_lens)]:
        assert np.array_equal(x, y)
    c = W.make_workload(2, seed=99)
    assert not np.array_equal(a.q, c.q)


def test_block_tables_use_distinct_pages_and_poison_the_rest():
    w = W.make_workload(5)
    used = []
    for b, L in enumerate(w.seq_lens):
        n = W.pages_for(L)
        assert np.all(w.block_tables[b, :n] >= 0)
        assert np.all(w.block_tables[b, n:] == -1)
        used.extend(w.block_tables[b, :n].tolist())
    assert len(used) == len(set(used))
    unused = np.setdiff1d(np.arange(w.num_pages), used)
    assert len(unused) > 0
    assert np.all(w.k_pool[unused] == W.BF16_NAN)
    # the slot the append will fill is poisoned in the pool and carried in k_new
    for b, L in enumerate(w.seq_lens):
        pos = L - 1
        page = w.block_tables[b, pos // W.PAGE_SIZE]
        assert np.all(w.k_pool[page, pos % W.PAGE_SIZE] == W.BF16_NAN)
        assert np.all(w.v_pool[page, pos % W.PAGE_SIZE] == W.BF16_NAN)
    assert np.all(w.k_new != W.BF16_NAN)


def test_workload_shapes_and_length_ranges():
    assert list(W.workload_seq_lens(1)) == [37]
    l2 = W.workload_seq_lens(2)
    assert l2.shape == (8,) and l2.min() >= 1 and l2.max() <= 2048
    l3 = W.workload_seq_lens(3)
    assert l3.shape == (64,) and l3.min() >= 16 and l3.max() <= 2048
    assert np.all(W.workload_seq_lens(4) == 2048)
    l5 = W.workload_seq_lens(5)
    assert l5.shape == (512,) and l5.min() >= 1 and l5.max() == 2048
    # clipped Zipf(1.1): a large share at the clip, some single-token sequences
    assert 0.3 < np.mean(l5 == 2048) < 0.6 and np.mean(l5 == 1) > 0.03
    # truncated Zipf(1.1): P(L = k) proportional to k^-1.1 on 1..2048 (mean of the law about
    # 179, worked out here from the definition), so few sequences are long
    k = np.arange(1, 2049, dtype=np.float64)
    law_mean = float((k ** -0.1).sum() / (k ** -1.1).sum())
    assert 175 < law_mean < 185
    l6 = W.workload_seq_lens(6)
    assert l6.shape == (512,) and l6.min() >= 1 and l6.max() <= 2048
    assert abs(l6.mean() - law_mean) < 60 and np.mean(l6 == 1) > 0.1
    assert np.array_equal(l6, W.workload_seq_lens(6))        # seeded


def test_small_workload_layout():
    w = W.make_workload(1)
    assert w.k_pool.shape == (64, 16, 8, 64) and w.q.shape == (1, 32, 64)
    assert list(w.block_tables[0, :3] >= 0) == [True] * 3 and w.block_tables[0, 3] == -1
    last = w.block_tables[0, 2]
    assert np.all(w.k_pool[last, 5:] == W.BF16_NAN) and not np.any(w.k_pool[last, :5] == W.BF16_NAN)


def test_placement_does_not_change_the_logical_cache():
    import oracle
    a = W.make_workload(2)
    b = W.make_workload(2, placement="identity")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.seq_lens, b.seq_lens)
    assert not np.array_equal(a.block_tables, b.block_tables)
    for i in range(a.batch):
        L = int(a.seq_lens[i])
        assert np.array_equal(oracle.gather_sequence(a.k_pool, a.block_tables[i], L),
                              oracle.gather_sequence(b.k_pool, b.block_tables[i], L))


# ---------------------------------------------------------------------------
# Sharp-score inputs: they must really raise a page-wise running maximum far
# past its first value, or the GPU tests built on them prove nothing about the
# rescale of the online softmax.
# ---------------------------------------------------------------------------
SHARP_LENS = [37, 100, 255, 256, 1000, 2047, 2048, 17, 1, 0]
RAISE_LOG2 = 8.0          # the decode kernel's lazy-rescale threshold, in log2 units


def _page_maxima_log2(w, b, h, k_pool, v_pool):
    """Per-page maxima of head h's scores of sequence b, in log2 units (float64)."""
    import oracle
    L = int(w.seq_lens[b])
    K = oracle.gather_sequence(k_pool, w.block_tables[b], L)[:, h // 4, :]
    q = oracle.bf16_bits_to_f64(w.q[b, h])
    s = w.scale * (K @ q) / np.log(2.0)
    return np.array([s[i:i + 16].max() for i in range(0, L, 16)])


def _rises(w, k_pool, v_pool):
    """(number of (sequence, head) whose running maximum rises by more than the
    threshold after the first page, spread of their page maxima)."""
    rises, spread = 0, 0.0
    for b in range(w.batch):
        if w.seq_lens[b] <= 16:
            continue
        for h in range(0, 32, 5):
            pm = _page_maxima_log2(w, b, h, k_pool, v_pool)
            if np.max(pm[1:]) > pm[0] + RAISE_LOG2:
                rises += 1
            spread = max(spread, float(pm.max() - pm.min()))
    return rises, spread


def test_sharp_inputs_raise_the_running_maximum_after_the_first_page():
    import oracle
    for mode in W.SHARP_MODES:
        w = W.make_sharp_batch(SHARP_LENS, 1200, 7, mode, append=True)
        k, v = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables,
                                w.seq_lens)
        rises, spread = _rises(w, k, v)
        if mode == "ramp_down":
            assert spread > RAISE_LOG2, mode        # split maxima far apart, largest first
        else:
            assert rises >= 5, (mode, rises)
            assert spread > 2 * RAISE_LOG2, (mode, spread)
    # the N(0, 1) workloads at scale 1/8 essentially never do (why these inputs exist)
    w = W.make_batch(SHARP_LENS, 1200, 7)
    assert _rises(w, w.k_pool, w.v_pool)[0] == 0


def test_sharp_tail_max_sits_on_the_appended_token_in_a_part_filled_page():
    import oracle
    w = W.make_sharp_batch(SHARP_LENS, 1200, 8, "tail_max", append=True)
    k, v = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.block_tables, w.seq_lens)
    for b, L in enumerate(w.seq_lens):
        if L < 2:
            continue
        K = oracle.gather_sequence(k, w.block_tables[b], int(L))
        for h in range(32):
            s = K[:, h // 4, :] @ oracle.bf16_bits_to_f64(w.q[b, h])
            assert int(np.argmax(s)) == L - 1, (b, h)
    assert any(L % 16 for L in SHARP_LENS if L)


def test_sharp_batch_layout_matches_make_batch_conventions():
    w = W.make_sharp_batch(SHARP_LENS, 1200, 9, "ramp_up", append=True)
    used = []
    for b, L in enumerate(w.seq_lens):
        n = W.pages_for(L)
        assert np.all(w.block_tables[b, n:] == -1)
        used.extend(w.block_tables[b, :n].tolist())
        if L:
            page = w.block_tables[b, (L - 1) // 16]
            assert np.all(w.k_pool[page, (L - 1) % 16] == W.BF16_NAN)
    assert len(used) == len(set(used))
    assert W.make_sharp_batch(SHARP_LENS, 1200, 9, "scale2").scale == W.SHARP_SCALE2
    rows = W.logical_rows(w.k_pool, w.block_tables[2], 254)
    assert rows.shape == (254, 8, 64) and not np.any(rows == W.BF16_NAN)
