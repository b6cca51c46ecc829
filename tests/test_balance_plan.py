"""The host plan of the balanced launch (include/pa_decode_balanced.h), on the CPU.

Every plan is decoded and checked against what the kernel assumes: each
(sequence, KV head) stream's pages are covered exactly once, in order, by
segments of wavefronts of ONE work-group; a stream split over wavefronts has
its first piece as the last segment of its wavefront and every later piece as
the first segment of the wavefronts `stride` apart; the wavefronts of one lane
(heads_together of them) hold the same pages of a sequence's consecutive heads;
no wavefront holds more than 7 segments or 256 pages; every idle sequence has
one zero-row segment; and the pages per work-group are balanced.  Planning
makes no HIP call (num_cus > 0).
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from paged_kv_decode_07_amd import binding as pa

HEADER, DESC, MAXSEG = 64, 64, 7


def decode_plan(plan, groups):
    assert plan[0] == 0x50414231 and plan[1] == groups and plan[4] == MAXSEG
    assert plan.size == HEADER + groups * 8 * DESC
    waves = []
    for k in range(groups):
        for w in range(8):
            d = plan[HEADER + (k * 8 + w) * DESC:][:DESC]
            segs = [tuple(int(x) for x in d[8 + 8 * j:][:8]) for j in range(int(d[0]))]
            waves.append((k, w, int(d[0]), int(d[1]), segs))
    return waves


def check_plan(lens, num_cus=256, max_blocks=128, h=8):
    lens = np.asarray(lens, np.int32)
    plan, groups = pa.balance_plan(lens, 1 << 20, max_blocks=max_blocks,
                                   max_seq_len=int(lens.max()) if lens.size else 0,
                                   num_cus=num_cus, heads_together=h, host_only=True)
    assert plan[5] == h
    waves = decode_plan(plan, groups)
    covered = {}
    idle = []
    byw = {(k, w): segs for k, w, _, _, segs in waves}
    load = np.zeros(groups, np.int64)
    for k, w, nseg, pages, segs in waves:
        assert 0 <= nseg <= MAXSEG and 0 <= pages <= 256
        assert pages == sum(x[3] - x[2] for x in segs)
        load[k] += pages
        for j, (b, g, p0, p1, L, kind, pieces, stride) in enumerate(segs):
            assert 0 <= b < len(lens) and L == lens[b]
            if g == 8:
                assert (p0, p1, kind, L) == (0, 0, 0, 0)
                idle.append(b)
                continue
            n = W.pages_for(L)
            assert 0 <= g < 8 and 0 <= p0 < p1 <= n <= max_blocks
            covered.setdefault((b, g), []).append((p0, p1, k, w, j, kind, pieces, stride))
            if kind == 1:
                assert j == nseg - 1 and pieces >= 2 and stride == h and w + (pieces - 1) * h < 8
            # the wavefronts of a lane hold the same pages of consecutive heads
            lane0 = byw[(k, w - w % h)]
            assert any(x[0] == b and x[2:4] == (p0, p1) and x[1] == g - w % h for x in lane0)
            if kind == 2:
                assert j == 0
    assert sorted(idle) == [b for b in range(len(lens)) if lens[b] == 0]
    for b in range(len(lens)):
        if lens[b] == 0:
            continue
        for g in range(8):
            parts = sorted(covered[(b, g)])
            # contiguous, complete, in one work-group, in consecutive wavefronts
            assert parts[0][0] == 0 and parts[-1][1] == W.pages_for(lens[b])
            assert all(x[1] == y[0] for x, y in zip(parts, parts[1:]))
            assert len({p[2] for p in parts}) == 1
            ws = [p[3] for p in parts]
            assert ws == list(range(ws[0], ws[0] + h * len(ws), h))
            if len(parts) == 1:
                assert parts[0][5] == 0
            else:
                assert h < 8
                assert parts[0][5] == 1 and parts[0][6] == len(parts)
                assert all(p[5] == 2 and p[4] == 0 for p in parts[1:])
                k = parts[0][2]
                for i in range(1, len(parts)):         # what the merger will read
                    sb, sg, *_ = byw[(k, parts[0][3] + i * h)][0]
                    assert (sb, sg) == (b, g)
    return groups, load


@pytest.mark.parametrize("h", [1, 2, 4, 8])
@pytest.mark.parametrize("wi", [1, 2, 3, 4, 5, 6])
def test_workload_plans_are_valid_and_balanced(wi, h):
    lens = W.workload_seq_lens(wi)
    groups, load = check_plan(lens, h=h)
    total = 8 * sum(W.pages_for(L) for L in lens)
    assert load.sum() == total
    if (wi in (4, 5) and h != 4) or (wi == 3 and h == 1):
        # units smaller than a work-group's share: within 5% of an even share
        # (with lanes of 4 heads the Zipf batch's short units need more than 7
        # pieces a wavefront in some groups, and the plan takes more groups)
        assert groups == 256
        assert load.max() <= 1.05 * total / groups + 8
    if wi == 4:
        assert load.min() == load.max() == 1024


def test_random_batches_and_edge_cases():
    rng = np.random.default_rng(5150)
    cases = [[0], [0, 0, 3], [1], [16, 17, 0, 2048], [2048] * 3, [1] * 700, [0] * 90 + [5],
             list(range(0, 2049, 37))]
    for _ in range(40):
        B = int(rng.integers(1, 600))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(0, 2049, size=B)
        elif kind == 1:
            lens = np.clip(rng.zipf(1.1, size=B), 1, 2048)
        else:
            lens = rng.choice([0, 1, 15, 16, 17, 2047, 2048], size=B)
        cases.append(list(lens))
    for lens in cases:
        for cus in (256, 80, 7):
            for h in (1, 2, 8):
                check_plan(lens, num_cus=cus, h=h)


def test_long_sequences_with_wide_tables():
    for h in (1, 2, 4):
        check_plan([4096, 3000, 1, 0, 4095], max_blocks=256, h=h)
    check_plan([4096, 3000, 17], max_blocks=256, h=8)   # 256 pages: one wavefront's most
    with pytest.raises(RuntimeError, match="VALUE"):      # 257 pages, whole per wavefront
        pa.balance_plan([4112, 3000], 1000, max_blocks=512, max_seq_len=4112, num_cus=256,
                        heads_together=8, host_only=True)


def test_refusals():
    with pytest.raises(RuntimeError, match="VALUE"):      # a length beyond max_seq_len
        pa.balance_plan([10, 50], 1000, max_seq_len=40, num_cus=256, host_only=True)
    with pytest.raises(RuntimeError, match="VALUE"):      # beyond the block table
        pa.balance_plan([3000], 1000, max_blocks=128, max_seq_len=2048, num_cus=256,
                        host_only=True)
    plan, groups = pa.balance_plan([], 10, max_seq_len=0, num_cus=256, host_only=True)
    assert groups >= 1 and plan.size == HEADER + groups * 8 * DESC
    with pytest.raises(RuntimeError, match="VALUE"):
        pa.balance_plan([10], 10, num_cus=256, heads_together=3, host_only=True)


def test_short_buffer_reports_the_size_and_every_word_is_written():
    import ctypes
    lib = pa.load_library()
    rng = np.random.default_rng(5)
    lens = np.ascontiguousarray(rng.integers(0, 2049, 300).astype(np.int32))
    shape = pa.make_shape(1 << 20, 128)
    words, groups = ctypes.c_int64(), ctypes.c_int32()
    args = (ctypes.byref(shape), lens.size, lens.ctypes.data_as(ctypes.c_void_p), 2048, 256, 1)
    short = np.zeros(HEADER + 8 * DESC, np.int32)
    assert lib.pa_balance_plan(*args, short.ctypes.data_as(ctypes.c_void_p), short.size,
                               ctypes.byref(words), ctypes.byref(groups)) == -6
    assert words.value == HEADER + groups.value * 8 * DESC and groups.value > 1
    assert (short == 0).all()                               # nothing written into a short buffer
    plans = []
    for fill in (0, -1, 0x5A5A5A5A):                        # whatever the buffer held before
        buf = np.full(words.value, fill, np.int32)
        assert lib.pa_balance_plan(*args, buf.ctypes.data_as(ctypes.c_void_p), buf.size,
                                   ctypes.byref(words), ctypes.byref(groups)) == 0
        plans.append(buf)
    assert all(np.array_equal(plans[0], p) for p in plans[1:])
    host, g = pa.balance_plan(lens, 1 << 20, max_seq_len=2048, num_cus=256, heads_together=1,
                              host_only=True)
    assert g == groups.value and np.array_equal(host, plans[0])


def test_wrapper_plans_beyond_its_first_guess():
    # many idle and one-page sequences need more work-groups than compute units
    lens = np.array([0] * 40 + [1] * 3000, np.int32)
    plan, groups = pa.balance_plan(lens, 1 << 20, max_seq_len=16, num_cus=8, heads_together=8,
                                   host_only=True)
    assert groups > 8 and plan.size == HEADER + groups * 8 * DESC
    check_plan(lens, num_cus=8, h=8)


def test_concurrent_planning_matches_sequential():
    # the planner keeps its buffers per calling thread; ctypes drops the GIL
    # during the call, so these plans are built concurrently
    import threading
    rng = np.random.default_rng(11)
    batches = [rng.integers(0, 2049, int(rng.integers(1, 600))).astype(np.int32) for _ in range(16)]
    hs = [1, 2, 4, 8]

    def plan(i):
        return pa.balance_plan(batches[i], 1 << 20, max_seq_len=2048, num_cus=256,
                               heads_together=hs[i % 4], host_only=True)
    want = [plan(i) for i in range(len(batches))]
    got = [[None] * len(batches) for _ in range(8)]

    def worker(t):
        for rep in range(3):
            for i in range(len(batches)):
                j = (i + t) % len(batches)
                got[t][j] = plan(j)
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for t in range(8):
        for i in range(len(batches)):
            assert got[t][i][1] == want[i][1] and np.array_equal(got[t][i][0], want[i][0])
