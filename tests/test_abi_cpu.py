"""The C-ABI library loads, exports what its header declares, and rejects bad
arguments on the host before any launch (no GPU needed: none of these calls
reaches the device)."""

import ctypes
import os
import re

import pytest

from paged_kv_decode_07_amd import binding as pa
from paged_kv_decode_07_amd import build as pb

import glob

HEADERS = sorted(glob.glob(os.path.join(pb.ROOT, "include", "*.h")))
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pb.LIB):
        pb.build()
    return pa.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(pa_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert "pa_append_kv" in names and "pa_decode_attention" in names
    assert set(names) == set(pa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.pa_abi_version() == 1


def test_status_strings(lib):
    for rc in range(0, -9, -1):
        s = pa.status_string(rc)
        assert s.startswith("PA_")
    assert "unknown" in pa.status_string(42)


def shape(**kw):
    s = pa.make_shape(64, 128)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def decode(lib, s, batch=1, max_seq_len=37, ptrs=None, scale=0.125, out_dtype=0, ps=1,
           ws=FAKE, ws_bytes=1 << 30, align_off=0):
    # every case here must be rejected (or be a batch-0 no-op) before a launch:
    # the pointers are fake.  With ps=1 the 37-token sequence needs 3 splits,
    # so a workspace is required and FAKE with ws_bytes=1<<30 is never reached
    # unless an earlier check fails first.
    p = ptrs or [ctypes.c_void_p(0x10000 + align_off)] * 6
    rc = lib.pa_decode_attention(ctypes.byref(s) if s is not None else None, batch,
                                   p[0], p[1], p[2], p[3], p[4], max_seq_len, scale, p[5],
                                   out_dtype, ps, ws, ws_bytes, None)
    assert rc < 0 or batch == 0, "a fake-pointer call was not rejected on the host"
    return rc


def test_decode_argument_errors(lib):
    assert decode(lib, None) == -1                                         # NULL shape
    assert decode(lib, shape(num_q_heads=16)) == -2                         # shape
    assert decode(lib, shape(head_dim=128)) == -2
    assert decode(lib, shape(page_size=32)) == -2
    assert decode(lib, shape(), batch=-1) == -6                             # value
    assert decode(lib, shape(), max_seq_len=2049) == -6
    assert decode(lib, shape(), scale=float("inf")) == -6
    assert decode(lib, shape(), out_dtype=7) == -6
    assert decode(lib, shape(), ps=129) == -6
    assert decode(lib, shape(), batch=0) == 0                               # no-op
    assert decode(lib, shape(), ptrs=[None] * 6) == -1                      # NULL tensors
    assert decode(lib, shape(), align_off=4) == -3                          # misaligned
    assert decode(lib, shape(), ws=None, ws_bytes=0) == -4                  # 3 splits need space
    assert decode(lib, shape(), ws_bytes=100) == -4


def test_workspace_sizes(lib):
    n = ctypes.c_size_t(0)
    s = shape()
    assert lib.pa_decode_workspace_bytes(ctypes.byref(s), 8, 2048, 128, ctypes.byref(n)) == 0
    assert n.value == 0                                                     # one split
    assert lib.pa_decode_workspace_bytes(ctypes.byref(s), 8, 2048, 16, ctypes.byref(n)) == 0
    rows = 8 * 8 * 32                                                       # B x splits x heads
    assert n.value == ((rows * 64 * 4 + 255) // 256) * 256 + rows * 2 * 4
    ps, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.pa_decode_plan(ctypes.byref(s), 8, 37, 2, ctypes.byref(ps), ctypes.byref(ns)) == 0
    assert (ps.value, ns.value) == (2, 2)


def test_append_argument_errors(lib):
    s = shape()
    F = FAKE
    assert lib.pa_append_kv(None, 1, F, F, F, F, F, F, None) == -1
    assert lib.pa_append_kv(ctypes.byref(shape(num_kv_heads=4)), 1, F, F, F, F, F, F, None) == -2
    assert lib.pa_append_kv(ctypes.byref(s), -2, F, F, F, F, F, F, None) == -6
    assert lib.pa_append_kv(ctypes.byref(s), 0, None, None, None, None, None, None, None) == 0
    assert lib.pa_append_kv(ctypes.byref(s), 1, None, F, F, F, F, F, None) == -1
    bad = ctypes.c_void_p(0x10008)
    assert lib.pa_append_kv(ctypes.byref(s), 1, bad, F, F, F, F, F, None) == -3
    assert lib.pa_append_kv(ctypes.byref(shape(num_pages=0)), 1, F, F, F, F, F, F, None) == -6


def test_validate_metadata_argument_errors(lib):
    s = shape()
    bad = ctypes.c_int64(0)
    assert lib.pa_validate_metadata(ctypes.byref(s), 0, None, None, 0, None,
                                    ctypes.byref(bad)) == 0
    assert lib.pa_validate_metadata(ctypes.byref(s), 2, None, None, 16, None,
                                    ctypes.byref(bad)) == -1


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        pa.load_library(str(tmp_path / "nope.so"))


def test_host_length_planner_choices():
    """The split plan for known lengths, for a 256-CU part, on the five workloads.

    Expected sizes are the fastest measured on MI355X for each workload, grid
    launch of the fused step (single sequence: one split of its 3 pages;
    workload 5: 205.1 us at 32 pages against 208.1 at 64 and 209.7 at 128).
    """
    import numpy as np
    import workloads as W
    expect = {1: 3, 2: 8, 3: 32, 4: 128, 5: 32}
    for i, ps_best in expect.items():
        lens = W.workload_seq_lens(i)
        ps, ns = pa.decode_plan_lengths(lens, 40000, num_cus=256)
        assert ps == ps_best, (i, ps)
        assert ns == -(-W.pages_for(int(lens.max())) // ps)
    # degenerate inputs
    assert pa.decode_plan_lengths(np.zeros(4, np.int32), 16, num_cus=256, max_seq_len=0) == (1, 1)
    s = pa.make_shape(64, 128)
    ps, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    lib = pa.load_library()
    assert lib.pa_decode_plan_lengths(ctypes.byref(s), 3, None, 16, 256, ctypes.byref(ps),
                                      ctypes.byref(ns)) == -1
    lens = (ctypes.c_int32 * 3)(1, 2, 3)
    assert lib.pa_decode_plan_lengths(ctypes.byref(s), 3, lens, 16, -1, ctypes.byref(ps),
                                      ctypes.byref(ns)) == -6


def decode_q8(lib, s, batch=1, max_seq_len=37, ptrs=None, scale=0.125, out_dtype=0, ps=1,
              ws=FAKE, ws_bytes=1 << 30, align_off=0, fused=False, sfx="_q8"):
    # as decode(): every case must be rejected before a launch (fake pointers);
    # sfx "_q8" or "_q4" picks the INT8 or the INT4 entry points
    n = 9 if fused else 7
    p = ptrs or [ctypes.c_void_p(0x10000 + align_off)] * n
    sp = ctypes.byref(s) if s is not None else None
    if fused:
        rc = getattr(lib, "pa_append_decode_attention" + sfx)(
            sp, batch, *p[:8], max_seq_len, scale, p[8], out_dtype, ps, ws, ws_bytes, None)
    else:
        rc = getattr(lib, "pa_decode_attention" + sfx)(
            sp, batch, *p[:6], max_seq_len, scale, p[6], out_dtype, ps, ws, ws_bytes, None)
    assert rc < 0 or batch == 0, "a fake-pointer call was not rejected on the host"
    return rc


@pytest.mark.parametrize("sfx", ["_q8", "_q4"])
@pytest.mark.parametrize("fused", [False, True])
def test_quant_decode_argument_errors(lib, fused, sfx):
    d = lambda *a, **k: decode_q8(lib, *a, fused=fused, sfx=sfx, **k)
    n = 9 if fused else 7
    assert d(None) == -1
    assert d(shape(num_kv_heads=4)) == -2
    assert d(shape(), batch=-1) == -6
    assert d(shape(), max_seq_len=2049) == -6
    assert d(shape(), scale=float("nan")) == -6
    assert d(shape(), out_dtype=3) == -6
    assert d(shape(), batch=0) == 0
    assert d(shape(), ptrs=[None] * n) == -1
    assert d(shape(), align_off=8) == -3
    assert d(shape(), ws=None, ws_bytes=0) == -4
    # the scale pool alone missing or misaligned
    p = [FAKE] * n
    p[(5 if fused else 3)] = None
    assert d(shape(), ptrs=p) == -1
    p[(5 if fused else 3)] = ctypes.c_void_p(0x10004)
    assert d(shape(), ptrs=p) == -3


@pytest.mark.parametrize("sfx", ["_q8", "_q4"])
def test_quant_append_and_fill_argument_errors(lib, sfx):
    fn = lambda name: getattr(lib, name + sfx)
    s, F = shape(), FAKE
    bad = ctypes.c_void_p(0x10008)
    assert fn("pa_append_kv")(None, 1, F, F, F, F, F, F, F, None) == -1
    assert fn("pa_append_kv")(ctypes.byref(shape(head_dim=32)), 1, F, F, F, F, F, F, F, None) == -2
    assert fn("pa_append_kv")(ctypes.byref(s), -1, F, F, F, F, F, F, F, None) == -6
    assert fn("pa_append_kv")(ctypes.byref(s), 0, None, None, None, None, None, None, None,
                               None) == 0
    assert fn("pa_append_kv")(ctypes.byref(s), 1, F, F, F, F, None, F, F, None) == -1
    assert fn("pa_append_kv")(ctypes.byref(s), 1, F, F, bad, F, F, F, F, None) == -3
    assert fn("pa_append_kv")(ctypes.byref(shape(num_pages=0)), 1, F, F, F, F, F, F, F,
                               None) == -6
    # RoPE variant: the tables are required
    assert fn("pa_append_kv_rope")(ctypes.byref(s), 1, F, F, F, None, F, F, F, F, F, F,
                                    None) == -1
    # fill
    assert fn("pa_fill_kv")(ctypes.byref(s), F, F, -1, 0, F, F, F, F, None) == -6
    assert fn("pa_fill_kv")(ctypes.byref(s), F, F, 10, 2040, F, F, F, F, None) == -6
    assert fn("pa_fill_kv")(ctypes.byref(s), F, F, 0, 0, None, None, None, None, None) == 0
    assert fn("pa_fill_kv")(ctypes.byref(s), F, F, 4, 0, F, F, F, None, None) == -1
    assert fn("pa_fill_kv")(ctypes.byref(s), F, F, 4, 0, F, F, bad, F, None) == -3


def test_q8_planner_choices():
    """The INT8 plan for known lengths on a 256-CU part, on workloads 2..5.

    Measured fastest split sizes for INT8 pages on MI355X: 8, 16, 128, 64
    pages; the fitted model picks 32 for workload 3, where it measured 1.6%
    slower than 16 (29.2 against 28.7 us).
    """
    import workloads as W
    expect = {2: 8, 3: 32, 4: 128, 5: 64}
    for i, ps_best in expect.items():
        lens = W.workload_seq_lens(i)
        ps, ns = pa.decode_plan_lengths_q8(lens, 40000, num_cus=256)
        assert ps == ps_best, (i, ps)
        assert ns == -(-W.pages_for(int(lens.max())) // ps)


def test_q4_planner_choices():
    """The INT4 cost model picks 8, 32, 128, 32 pages for workloads 2-5.

    It allows two work-groups per CU for even batches, and a launch whose work-groups all
    fit the CUs runs two wavefronts per KV head.  At workload 4, one 128-page split per
    sequence then streams with two wavefronts per head and no split merge.
    """
    import workloads as W
    expect = {2: 8, 3: 32, 4: 128, 5: 32}
    for i, ps_best in expect.items():
        lens = W.workload_seq_lens(i)
        ps, ns = pa.decode_plan_lengths_q4(lens, 40000, num_cus=256)
        assert ps == ps_best, (i, ps)
        assert ns == -(-W.pages_for(int(lens.max())) // ps)


def test_stream_read_argument_errors(lib):
    F, sink = FAKE, ctypes.c_void_p(0x20000)
    assert lib.pa_stream_read(None, 1024, sink, 0, None) == -1
    assert lib.pa_stream_read(F, 1024, None, 0, None) == -1
    assert lib.pa_stream_read(ctypes.c_void_p(0x10008), 1024, sink, 0, None) == -3
    assert lib.pa_stream_read(F, 1000, sink, 0, None) == -6          # not a multiple of 16
    assert lib.pa_stream_read(F, 0, sink, 0, None) == -6
    assert lib.pa_stream_read(F, 1024, sink, -1, None) == -6
    assert lib.pa_stream_read(F, 1024, sink, 65537, None) == -6


def test_page_stream_argument_errors(lib):
    F, T, sink = FAKE, ctypes.c_void_p(0x30000), ctypes.c_void_p(0x20000)
    good = pa.make_shape(64, 8)

    def call(shape=good, batch=2, k=F, v=F, s=F, fmt=0, bt=T, lens=T, wph=1, ring=2, out=sink):
        return lib.pa_page_stream(ctypes.byref(shape) if shape is not None else None, batch, k, v,
                                  s, fmt, bt, lens, wph, ring, out, None)
    assert call(batch=0) == 0                                  # nothing to stream, no launch
    assert call(shape=None) == -1
    assert call(shape=pa.make_shape(64, 8, head_dim=128)) == -2
    assert call(shape=pa.make_shape(64, 257)) == -6            # beyond the 256-page window
    for bad in (dict(fmt=3), dict(fmt=-1), dict(wph=0), dict(wph=3), dict(ring=0), dict(ring=4),
                dict(batch=-1)):
        assert call(**bad) == -6, bad
    assert call(fmt=0, wph=2, ring=3) == -6                    # 192 KiB of LDS ring
    for null in (dict(k=None), dict(v=None), dict(bt=None), dict(lens=None), dict(out=None),
                 dict(fmt=1, s=None), dict(fmt=2, s=None)):
        assert call(**null) == -1, null
    assert call(k=ctypes.c_void_p(0x10008)) == -3
    assert call(fmt=1, s=ctypes.c_void_p(0x10004)) == -3
    assert call(lens=ctypes.c_void_p(0x30002)) == -3


def test_timeline_argument_errors(lib):
    F, T = FAKE, ctypes.c_void_p(0x30000)
    good = pa.make_shape(64, 8)

    def call(shape=good, batch=2, fmt=0, s=None, groups=2, plan_words=1 << 20,
             stamps=ctypes.c_void_p(0x40000), words=2 * 8 * 8):
        return lib.pa_decode_balanced_timeline(
            ctypes.byref(shape) if shape is not None else None, batch, F, None, None, F, F, s,
            fmt, T, T, 16, ctypes.c_float(0.125), F, F, plan_words, groups, stamps, words, None)
    assert call(stamps=None) == -1
    assert call(stamps=ctypes.c_void_p(0x40004)) == -3         # 8-byte words
    assert call(words=2 * 8 * 8 - 1) == -6                     # 8 words per wavefront
    assert call(groups=0) == -6
    assert call(batch=0) == 0                                  # nothing to launch
    assert call(shape=None) == -1
    assert call(shape=pa.make_shape(64, 8, head_dim=128)) == -2
    assert call(fmt=3) == -6
    assert call(fmt=1) == -1                                   # INT8 pages need their scales
    assert call(plan_words=64) == -6                           # plan shorter than its groups
    assert lib.pa_wall_clock_khz(None) == -1


def test_balanced_launch_refuses_page_ids_beyond_28_bits(lib):
    F = FAKE
    shape = pa.make_shape((1 << 28) + 1, 128)      # checked before the plan and any launch
    rc = lib.pa_decode_balanced(ctypes.byref(shape), 1, F, None, None, None, F, F, None, 0,
                                F, F, 16, ctypes.c_float(0.125), F, 0, F, 1 << 20, 1, None)
    assert rc == -6


def test_worklist_covers_every_item_once_largest_first():
    import numpy as np
    lens = np.array([0, 1, 2048, 17, 300, 2049, 16, 33, 1000], np.int32)    # 2049: beyond the bound
    for ps in (1, 3, 8, 128):
        work, ps_out, ns = pa.decode_worklist(lens, 40000, max_seq_len=2048, pages_per_split=ps)
        assert ps_out == ps and ns == -(-128 // ps)
        pages = lambda b: -(-int(lens[b]) // 16) if 0 < lens[b] <= 2048 else 0
        want = set()
        for b in range(len(lens)):
            n = pages(b)
            want |= {(b, k) for k in range(max(1, -(-n // ps)))}
        got = [tuple(x) for x in work.tolist()]
        assert len(got) == len(set(got)) and set(got) == want
        size = [min(ps, pages(b) - s * ps) if pages(b) else 0 for b, s in got]
        assert size == sorted(size, reverse=True)
        # ties keep the (sequence, split) order
        for (b0, s0), (b1, s1), z0, z1 in zip(got, got[1:], size, size[1:]):
            if z0 == z1:
                assert (b0, s0) < (b1, s1)


def test_worklist_capacity_and_arguments(lib):
    import numpy as np
    lens = (ctypes.c_int32 * 3)(100, 200, 300)
    s = pa.make_shape(64, 128)
    work = (ctypes.c_int32 * 4)()
    count, ps, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    # 3 sequences x 19 pages at 1 page per split need more than 2 items
    assert lib.pa_decode_worklist(ctypes.byref(s), 3, lens, 300, 1, 0, 0, work, 2,
                                  ctypes.byref(count), ctypes.byref(ps), ctypes.byref(ns)) == -6
    assert count.value == 7 + 13 + 19
    big = (ctypes.c_int32 * 80)()
    for fmt in (0, 1, 2):
        assert lib.pa_decode_worklist(ctypes.byref(s), 3, lens, 300, 1, fmt, 0, big, 40,
                                      ctypes.byref(count), None, None) == 0
    for fmt in (-1, 3):
        assert lib.pa_decode_worklist(ctypes.byref(s), 3, lens, 300, 1, fmt, 0, big, 40,
                                      ctypes.byref(count), None, None) == -6     # bad format
    assert lib.pa_decode_worklist(ctypes.byref(s), 3, None, 300, 1, 0, 0, work, 2,
                                  ctypes.byref(count), None, None) == -1
    F = FAKE
    # a work list needs an explicit split size and at least one item
    assert lib.pa_append_decode_attention_worklist(
        ctypes.byref(s), 1, F, F, F, F, F, F, F, 37, 0.125, F, 0, 0, F, 4, F, 1 << 30, None) == -6
    assert lib.pa_append_decode_attention_worklist(
        ctypes.byref(s), 1, F, F, F, F, F, F, F, 37, 0.125, F, 0, 2, F, 0, F, 1 << 30, None) == -6
    assert lib.pa_append_decode_attention_worklist(
        ctypes.byref(s), 1, F, F, F, F, F, F, F, 37, 0.125, F, 0, 2, None, 4, F, 1 << 30, None) == -1
    for sfx in ("_q8", "_q4"):
        assert getattr(lib, "pa_append_decode_attention_worklist" + sfx)(
            ctypes.byref(s), 1, F, F, F, F, F, F, F, F, 37, 0.125, F, 0, 0, F, 4, F, 1 << 30,
            None) == -6


def test_worklist_planner_choices():
    """Split sizes planned for work-list launches on a 256-CU part (measured fastest on MI355X
    among 8..128 for workloads 2, 3 and 5, BF16 and INT8 pages alike: 8, 16, 32-64; the even
    batch 4 keeps one 128-page split per sequence)."""
    import workloads as W
    expect = {2: 8, 3: 16, 4: 128, 5: 64}
    for i, ps_best in expect.items():
        lens = W.workload_seq_lens(i)
        for int8 in (False, True):
            work, ps, ns = pa.decode_worklist(lens, 40000, num_cus=256, int8=int8)
            assert ps == ps_best, (i, int8, ps)


def test_c_client_is_built_and_rejects_bad_input(tmp_path):
    """The C-ABI client links against the library; malformed input exits 2 before any HIP call."""
    import subprocess
    client = pb.CLIENT
    if not os.path.exists(client):
        pb.build_client()
    assert subprocess.run([client], capture_output=True).returncode == 2
    assert subprocess.run([client, str(tmp_path)], capture_output=True).returncode == 2


def test_noalloc_entry_point_refuses_on_the_host(lib):
    """The allocation-free fused step checks its arguments and the size of the
    plan's partials against its fixed scratch before touching any device."""
    f = lib.pa_append_decode_attention_noalloc
    P = FAKE

    def call(s, batch, max_seq_len, ps, k_new=P, out_dtype=0, scale=0.125):
        return f(ctypes.byref(s) if s is not None else None, batch, P, k_new, P, P, P, P, P,
                 max_seq_len, scale, P, out_dtype, ps, None)
    assert call(shape(), 0, 37, 1) == 0                            # batch 0: nothing to do
    assert call(None, 1, 37, 1) == -1                              # PA_ERR_NULL
    assert call(shape(), 1, 37, 1, k_new=None) == -1
    assert call(shape(num_q_heads=16), 1, 37, 1) == -2             # PA_ERR_SHAPE
    assert call(shape(), 1, 5000, 1) == -6                         # PA_ERR_VALUE: beyond the table
    assert call(shape(), 1, 37, 300) == -6                         # split larger than 256 pages
    # partials larger than the scratch: 8192 sequences x 16 splits of 8 pages
    need = ctypes.c_size_t()
    assert lib.pa_decode_workspace_bytes(ctypes.byref(shape()), 8192, 2048, 8,
                                         ctypes.byref(need)) == 0
    assert need.value > pa.NOALLOC_SCRATCH_BYTES
    assert call(shape(), 8192, 2048, 8) == -4                      # PA_ERR_WORKSPACE
    assert pa.NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(os.path.join(pb.ROOT, "include", "pa_decode.h")).read()
    assert "#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text
