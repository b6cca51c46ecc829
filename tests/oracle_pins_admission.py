"""Pins for the reference page allocator and admission control.

Expected values are the credit rule worked by hand on chosen requests, the
pool sizes the engine's README states (128 MiB default pool of 32 KiB pages,
16 layers, 2,048-token context) and invariants of any valid allocator.
Each pin takes a module exposing ``PagePool`` (the oracle, or a copy with a
planted mistake).
"""

from __future__ import annotations

import numpy as np

DEFAULT_POOL_PAGES = 4096          # 128 MiB / 32 KiB
LAYERS = 16


def pin_credit_rule_by_hand(m):
    pool = m.PagePool(DEFAULT_POOL_PAGES)
    # prompt 100 + 29 new - 1 = 128 tokens = 8 pages per layer, 16 layers
    assert pool.credit_for(100, 29) == (29, 128)
    # output budget capped by the context: 2000 + min(500, 48) - 1 = 2047 tokens = 128 pages
    assert pool.credit_for(2000, 500) == (48, 2048)
    # a single prompt token and one new token: 1 processed token = 1 page per layer
    assert pool.credit_for(1, 1) == (1, 16)
    # 16 + 2 - 1 = 17 tokens: 2 pages per layer
    assert pool.credit_for(16, 2) == (2, 32)


def pin_default_pool_holds_exactly_two_full_context_requests(m):
    pool = m.PagePool(DEFAULT_POOL_PAGES)
    for rid in range(3):
        assert pool.submit(rid, 1, 4096) == m.WAIT       # each: 2047 tokens, 2048 pages
    assert pool.admit() == [0, 1]
    assert pool.stats["admission_waits"] == 1
    # short requests are not capped at two
    pool2 = m.PagePool(DEFAULT_POOL_PAGES)
    for rid in range(10):
        pool2.submit(rid, 20, 64)                        # 83 tokens: 6 pages x 16 = 96
    assert pool2.admit() == list(range(10))


def pin_small_pool_queues_and_rejects(m):
    pool = m.PagePool(256)                               # 8 MiB of 32 KiB pages
    for rid in range(3):
        pool.submit(rid, 20, 64)                         # 96 pages each
    assert pool.admit() == [0, 1]
    assert pool.submit(9, 1000, 64) == m.REJECT          # 1063 tokens: 67 x 16 = 1072 > 256
    assert pool.submit(10, 2048, 1) == m.REJECT          # prompt leaves no room in the context
    pool.finish(0)
    assert pool.admit() == [2]


def pin_fifo_no_overtaking(m):
    pool = m.PagePool(256)
    pool.submit(0, 20, 64)                               # 96
    pool.submit(1, 200, 40)                              # 239 tokens: 15 x 16 = 240
    pool.submit(2, 1, 1)                                 # 16, would fit, must wait behind 1
    assert pool.admit() == [0]
    assert pool.admit() == []
    pool.finish(0)
    assert pool.admit() == [1, 2]


def pin_static_mode_waits_for_the_group(m):
    pool = m.PagePool(256, static=True)
    pool.submit(0, 20, 64)
    pool.submit(1, 20, 64)
    pool.submit(2, 20, 64)
    assert pool.admit() == [0, 1]
    pool.finish(0)
    assert pool.admit() == []                            # 1 still running
    pool.finish(1)
    assert pool.admit() == [2]


def pin_lazy_pages_lowest_free_first(m):
    pool = m.PagePool(64, num_layers=2)
    pool.submit(0, 30, 10)                               # 39 tokens: 3 pages x 2 layers
    pool.submit(1, 5, 3)                                 # 7 tokens: 1 page x 2 layers
    assert pool.admit() == [0, 1]
    pool.grow(0, 30)                                     # prompt: 2 pages per layer
    assert pool.block_table(0, 0) == [0, 1] and pool.block_table(0, 1) == [2, 3]
    pool.grow(1, 5)
    assert pool.block_table(1, 0) == [4] and pool.block_table(1, 1) == [5]
    pool.grow(0, 32)                                     # still 2 pages
    assert pool.stats["free_pages"] == 64 - 6
    pool.grow(0, 33)                                     # third page in each layer
    assert pool.block_table(0, 0) == [0, 1, 6] and pool.block_table(0, 1) == [2, 3, 7]
    pool.finish(1)
    pool.submit(2, 3, 2)
    assert pool.admit() == [2]
    pool.grow(2, 4)
    assert pool.block_table(2, 0) == [4] and pool.block_table(2, 1) == [5]
    assert pool.stats["peak_allocated"] == 8


def pin_random_trace_invariants(m):
    rng = np.random.default_rng(401)
    pool = m.PagePool(300, num_layers=4)
    next_id, live = 0, {}
    for _ in range(400):
        op = rng.integers(0, 4)
        if op == 0:
            prompt = int(rng.integers(1, 300)); mx = int(rng.integers(1, 200))
            res = pool.submit(next_id, prompt, mx)
            assert res in (m.WAIT, m.REJECT)
            next_id += 1
        elif op == 1:
            for rid in pool.admit():
                r = pool.active[rid]
                live[rid] = r.prompt
                pool.grow(rid, r.prompt)
        elif op == 2 and live:
            rid = list(live)[int(rng.integers(0, len(live)))]
            r = pool.active[rid]
            if r.length < r.prompt + r.allowed_new - 1:
                pool.grow(rid, r.length + 1)
            pool.step()
        elif op == 3 and live:
            rid = list(live)[int(rng.integers(0, len(live)))]
            pool.finish(rid)
            del live[rid]
        held = [p for r in pool.active.values() for lp in r.pages for p in lp]
        assert len(held) == len(set(held))
        assert len(held) + len(pool.free) == pool.num_pages
        assert set(held).isdisjoint(pool.free)
        assert pool.reserved == sum(r.credit for r in pool.active.values()) <= pool.num_pages
        for r in pool.active.values():
            assert sum(len(lp) for lp in r.pages) <= r.credit


ALL_ADMISSION_PINS = [
    pin_credit_rule_by_hand,
    pin_default_pool_holds_exactly_two_full_context_requests,
    pin_small_pool_queues_and_rejects,
    pin_fifo_no_overtaking,
    pin_static_mode_waits_for_the_group,
    pin_lazy_pages_lowest_free_first,
    pin_random_trace_invariants,
]
