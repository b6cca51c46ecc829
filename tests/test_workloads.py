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
