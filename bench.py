#!/usr/bin/env python3
"""Benchmark of the paged GQA decode hot path on one MI355X.

One step = one layer's decode step of the full-context batch: the one-token
page append of every sequence and paged GQA decode attention (32 query heads
over 8 KV heads, head_dim 64, BF16 K/V in 16-token pages, FP32 online
softmax), including the split merge when the plan has one.  The step is the
library's fused single-launch call (pa_append_decode_attention); the same
step as two calls (pa_append_kv then pa_decode_attention) is timed as well.
Workload: batch 256, every sequence 2,048 tokens after the append (128 pages
each, 1 GiB of K/V), pages at seeded-random places in a pool of exactly
32,768 pages; synthetic BF16 N(0, 1) data.

Timing: the inputs are resident in HBM before the timed region.  Before each
step a separate 1 GiB buffer is read (a reduction), so the step starts with
L2 and Infinity Cache holding none of its inputs; the flush only reads, so it
leaves no dirty lines whose write-back would land inside the next step.
Pass A times the K steps with one event pair around each step; pass B
repeats them with the library recording events right around its main
kernel (the roofline figure); pass C times the two-call form; pass D the
fused step with RoPE; pass E the fused step over INT8 pages and pass F over
INT4 pages (the BF16 cache quantised on the GPU first).  Two diagnostics follow: the same step with the
pages in identity order, and a plain streaming read of 1 GiB (the achievable
read bandwidth, beside the published peak).  The flush is outside every event
pair.  The oracle baseline runs on one core and on a pool of worker processes
forked before the GPU is initialised.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attention KV-read GB/s (% of MI355X HBM peak) + sequences/s per layer"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic_b256_l2048.json")
TRAFFIC_FILE_Q8 = os.path.join(ROOT, "profiles", "decode_q8_kernel_traffic_b256_l2048.json")
TRAFFIC_FILE_Q4 = os.path.join(ROOT, "profiles", "decode_q4_kernel_traffic_b256_l2048.json")
_CSRC = os.path.join(ROOT, "paged_kv_decode_07_amd", "csrc")
_DEVICE = ("pa_kernels.h", "pa_kernels_q8.h", "pa_decode_kernel.h", "pa_host.h")
KERNEL_SOURCES = [os.path.join(_CSRC, n) for n in _DEVICE + ("pa_decode.hip",)]
KERNEL_SOURCES_Q8 = [os.path.join(_CSRC, n) for n in _DEVICE + ("pa_decode_q8.hip",)]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str = TRAFFIC_FILE, sources=None):
    """HBM bytes per launch of a kernel from committed rocprofv3 counters.

    The summary holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    kernel and of a device copy of known size, taken on the same kernel
    source; None when absent or when the kernel has changed since.
    """
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash(sources):
        return None
    return int(round(t["hbm_bytes_per_launch"]))


_CPU_STATE = None          # (batch, k_ref, v_ref): set before the pool forks


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def _oracle_decodes(first: int, stride: int, seconds: float, gpu_out=None):
    """Decode sequences first, first+stride, ... (cycling) with the oracle for ``seconds``."""
    import numpy as np
    import oracle
    batch, k_ref, v_ref = _CPU_STATE
    done, worst, t0 = [], 0.0, time.perf_counter()
    while True:
        b = (first + stride * len(done)) % batch.batch
        ref = oracle.decode_attention(batch.q, k_ref, v_ref, batch.block_tables,
                                      batch.seq_lens, batch.scale, sequences=[b])
        if gpu_out is not None:
            worst = max(worst, float(np.max(np.abs(ref[b] - gpu_out[b]))))
        done.append(b)
        if time.perf_counter() - t0 >= seconds and len(done) >= 2:
            break
    return done, time.perf_counter() - t0, worst


def _pool_leg(args):
    first, stride, seconds = args
    done, dt, _ = _oracle_decodes(first, stride, seconds)
    return done, dt


def prepare_cpu_baseline(batch, pool_workers: int):
    """Append on the host and fork the worker pool, before the GPU is initialised
    (the workers inherit the inputs and never touch the GPU)."""
    global _CPU_STATE
    import multiprocessing as mp
    import oracle
    k_ref, v_ref = oracle.append_kv(batch.k_pool, batch.v_pool, batch.k_new, batch.v_new,
                                    batch.block_tables, batch.seq_lens)
    _CPU_STATE = (batch, k_ref, v_ref)
    if pool_workers <= 1:
        return None
    return mp.get_context("fork").Pool(pool_workers, initializer=_blas_one_thread)


def cpu_baseline(gpu_out, seconds: float, pool=None, pool_workers: int = 0):
    """The oracle, as it stands, over the same workload: one core, then a process pool."""
    import contextlib
    batch = _CPU_STATE[0]
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = contextlib.nullcontext()
    with limit:
        done, dt, worst = _oracle_decodes(0, 1, seconds, gpu_out)
    tokens = int(sum(int(batch.seq_lens[b]) for b in done))
    kv = tokens * 2048
    res = {
        "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{len(done)} sequence decodes cycling over the {batch.batch} sequences "
                   f"({tokens} tokens, {kv / 2**20:.0f} MiB of K/V), float64 NumPy, "
                   f"1 BLAS thread, {dt:.1f} s"),
        "seq_per_s": round(len(done) / dt, 3),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": 1,
        "max_abs_vs_gpu_on_sample": worst,
    }
    if pool is not None:
        t0 = time.perf_counter()
        legs = pool.map(_pool_leg, [(w, pool_workers, seconds) for w in range(pool_workers)])
        wall = time.perf_counter() - t0
        n = sum(len(d) for d, _ in legs)
        ptok = sum(int(batch.seq_lens[b]) for d, _ in legs for b in d)
        res["pool"] = {
            "value": round(ptok * 2048 / wall / 1e9, 4), "unit": "GB/s", "cores": pool_workers,
            "sample": (f"{n} sequence decodes over {pool_workers} worker processes "
                       f"(1 BLAS thread each), {wall:.1f} s wall"),
            "seq_per_s": round(n / wall, 3),
        }
    return res


def run_sweep(args) -> int:
    """Every workload's fused append + attention step (one layer; workload 3 is its
    first layer), cold caches, medians of ``--steps`` event-timed steps."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)
    flush_out = torch.empty((), dtype=torch.int32, device=dev)
    workspace = torch.empty(256 << 20, dtype=torch.uint8, device=dev)

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def timed(fn, n):
        for _ in range(max(args.warmup, 1)):
            fn()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            if not args.no_flush:
                torch.amax(flush_buf, dim=None, out=flush_out)
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3

    for wi in (1, 2, 3, 4, 5):
        t0 = time.perf_counter()
        w = W.make_workload(wi, append=True)
        log(f"workload {wi}: {w.batch} sequences, {w.num_pages} pages "
            f"(generated in {time.perf_counter() - t0:.1f} s)")
        q, kp, vp = up16(w.q), up16(w.k_pool), up16(w.v_pool)
        kn, vn = up16(w.k_new), up16(w.v_new)
        bt = torch.from_numpy(w.block_tables).to(dev)
        lens = torch.from_numpy(w.seq_lens).to(dev)
        out = torch.empty((w.batch, 32, 64), dtype=torch.float32, device=dev)
        npg, msl = w.num_pages, w.max_seq_len
        ident = torch.arange(npg, dtype=torch.int32, device=dev)
        kc, vc, sc = pa.new_q8_pools(npg, device=dev)
        pa.fill_kv_q8(kp.view(npg * 16, 8, 64), vp.view(npg * 16, 8, 64), ident, 0, kc, vc, sc,
                      stream=stream)
        kc4, vc4, sc4 = pa.new_q4_pools(npg, device=dev)
        pa.fill_kv_q4(kp.view(npg * 16, 8, 64), vp.view(npg * 16, 8, 64), ident, 0, kc4, vc4,
                      sc4, stream=stream)
        formats = {"bf16": (A.step_bytes, pa.decode_plan_lengths, (kp, vp), None),
                   "int8": (A.step_bytes_q8, pa.decode_plan_lengths_q8, (kc, vc), sc),
                   "int4": (A.step_bytes_q4, pa.decode_plan_lengths_q4, (kc4, vc4), sc4)}
        for fmt, (acct, plan, (kpool, vpool), scales) in formats.items():
            kv = acct(w.seq_lens, append=True)["kv"]
            ps, ns = plan(w.seq_lens, npg, max_seq_len=msl)
            cases = []
            if fmt == "bf16":
                cases.append(("grid (lengths plan)", ps, ns, lambda ps=ps: pa.append_decode_attention(
                    q, kn, vn, kp, vp, bt, lens, msl, scale=w.scale, out=out,
                    pages_per_split=ps, workspace=workspace, stream=stream)))
            else:
                fused = pa.append_decode_attention_q8 if fmt == "int8" else pa.append_decode_attention_q4
                cases.append(("grid (lengths plan)", ps, ns,
                              lambda ps=ps, fused=fused, kpool=kpool, vpool=vpool, scales=scales:
                              fused(q, kn, vn, kpool, vpool, scales, bt, lens, msl, scale=w.scale,
                                    out=out, pages_per_split=ps, workspace=workspace,
                                    stream=stream)))
            if w.batch > 1:
                wl, wps, _ = pa.decode_worklist(w.seq_lens, npg, max_seq_len=msl,
                                                int8=fmt == "int8", int4=fmt == "int4")
                wd = torch.from_numpy(wl).to(dev)
                cases.append(("work list", wps, len(wl),
                              lambda wd=wd, wps=wps, kpool=kpool, vpool=vpool, scales=scales:
                              pa.append_decode_attention_worklist(
                                  q, kn, vn, kpool, vpool, bt, lens, msl, wd, wps, scale=w.scale,
                                  out=out, workspace=workspace, stream=stream, kv_scales=scales)))
            for launch, cps, units, fn in cases:
                t = timed(fn, args.steps)
                print(json.dumps({
                    "workload": wi, "desc": W.WORKLOADS[wi], "pages": fmt,
                    "launch": launch, "pages_per_split": int(cps),
                    ("items" if launch == "work list" else "splits"): int(units),
                    "step_us": round(t * 1e6, 2), "kv_bytes": int(kv),
                    "kv_gbps": round(kv / t / 1e9, 1),
                    "seq_per_s_per_layer": round(int(np.count_nonzero(w.seq_lens)) / t, 1)}),
                    flush=True)
        del q, kp, vp, kn, vn, bt, lens, out, kc, vc, sc, kc4, vc4, sc4, formats, cases
        torch.cuda.empty_cache()

    # workload 3 as a model step: the 16 layers' fused steps back to back (one
    # pool region per layer), launched one by one and replayed as a HIP graph
    layers = []
    t0 = time.perf_counter()
    for layer in range(16):
        w = W.make_workload(3, layer=layer, append=True)
        layers.append(dict(q=up16(w.q), kp=up16(w.k_pool), vp=up16(w.v_pool), kn=up16(w.k_new),
                           vn=up16(w.v_new), bt=torch.from_numpy(w.block_tables).to(dev),
                           lens=torch.from_numpy(w.seq_lens).to(dev),
                           out=torch.empty((w.batch, 32, 64), dtype=torch.float32, device=dev)))
    log(f"workload 3, 16 layers generated in {time.perf_counter() - t0:.1f} s")
    w0 = W.make_workload(3, layer=0, append=True)
    ps, ns = pa.decode_plan_lengths(w0.seq_lens, w0.num_pages, max_seq_len=w0.max_seq_len)
    kv16 = 16 * A.step_bytes(w0.seq_lens, append=True)["kv"]

    wl, wps, _ = pa.decode_worklist(w0.seq_lens, w0.num_pages, max_seq_len=w0.max_seq_len)
    wd = torch.from_numpy(wl).to(dev)

    def model_step(st, worklist):
        for L in layers:
            if worklist:
                pa.append_decode_attention_worklist(
                    L["q"], L["kn"], L["vn"], L["kp"], L["vp"], L["bt"], L["lens"],
                    w0.max_seq_len, wd, wps, scale=w0.scale, out=L["out"], workspace=workspace,
                    stream=st)
            else:
                pa.append_decode_attention(L["q"], L["kn"], L["vn"], L["kp"], L["vp"], L["bt"],
                                           L["lens"], w0.max_seq_len, scale=w0.scale,
                                           out=L["out"], pages_per_split=ps, workspace=workspace,
                                           stream=st)

    for worklist in (False, True):
        t_eager = timed(lambda: model_step(stream, worklist), args.steps)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                model_step(side, worklist)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        t_graph = timed(graph.replay, args.steps)
        base = "work list" if worklist else "grid (lengths plan)"
        for launch, t in ((f"{base}, 16 calls", t_eager), (f"{base}, HIP graph of 16 calls", t_graph)):
            print(json.dumps({
                "workload": 3, "desc": W.WORKLOADS[3] + " (all 16 layers)", "pages": "bf16",
                "launch": launch, "pages_per_split": int(wps if worklist else ps),
                ("items" if worklist else "splits"): int(len(wl) if worklist else ns),
                "step_us": round(t * 1e6, 2), "kv_bytes": int(kv16),
                "kv_gbps": round(kv16 / t / 1e9, 1),
                "seq_per_s": round(int(np.count_nonzero(w0.seq_lens)) / t, 1)}), flush=True)
        del graph
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pages-per-split", type=int, default=0, help="0 = library plan")
    ap.add_argument("--placement", choices=["random", "identity"], default="random")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle process-pool size (0 = the CPUs this process may use, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a 256 MiB device copy per step (outside the timed events), "
                         "the known-size reference for hardware byte counters")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: time the fused step of every workload "
                         "(1-5), BF16 and INT8 pages, grid launch with the library plan and "
                         "work-list launch; one JSON line per case")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X "
              "and has no multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads as W
    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    if args.sweep:
        return run_sweep(args)

    t0 = time.perf_counter()
    batch = W.make_workload(4, placement=args.placement, append=True)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s "
        f"({batch.batch} sequences, {batch.num_pages} pages)")
    pool, pool_workers = None, 0
    if not args.no_cpu_baseline:
        pool_workers = args.cpu_workers or min(len(os.sched_getaffinity(0)), 16)
        pool = prepare_cpu_baseline(batch, pool_workers)

    # the GPU is first touched here, after the oracle's worker processes were forked
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    q, k_pool, v_pool = up16(batch.q), up16(batch.k_pool), up16(batch.v_pool)
    k_new, v_new = up16(batch.k_new), up16(batch.v_new)
    bt = torch.from_numpy(batch.block_tables).to(dev)
    lens = torch.from_numpy(batch.seq_lens).to(dev)
    B, msl = batch.batch, batch.max_seq_len
    ps, ns = pa.decode_plan(B, msl, batch.num_pages, 128, args.pages_per_split)
    ws_bytes = pa.decode_workspace_bytes(B, msl, batch.num_pages, 128, ps)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((B, 32, 64), dtype=torch.float32, device=dev)
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)       # 1 GiB, read only
    flush_out = torch.empty((), dtype=torch.int32, device=dev)

    def flush():
        torch.amax(flush_buf, dim=None, out=flush_out)
    stream = torch.cuda.current_stream()
    log(f"plan: {ps} pages per split, {ns} splits; workspace {ws_bytes} B")
    if args.calibration_copy:
        copy_src = torch.ones(2**26, dtype=torch.int32, device=dev)     # 256 MiB
        copy_dst = torch.empty_like(copy_src)

    K, Wm = args.steps, args.warmup

    def step(marks=None):
        pa.append_decode_attention(q, k_new, v_new, k_pool, v_pool, bt, lens, msl,
                                   scale=batch.scale, out=out, pages_per_split=ps,
                                   workspace=workspace, stream=stream,
                                   event_before_main=marks[0] if marks else None,
                                   event_after_main=marks[1] if marks else None)

    def two_call_step():
        pa.append_kv(k_new, v_new, k_pool, v_pool, bt, lens, stream=stream)
        pa.decode_attention(q, k_pool, v_pool, bt, lens, msl, scale=batch.scale, out=out,
                            pages_per_split=ps, workspace=workspace, stream=stream)

    def pre_step():
        if args.calibration_copy:
            copy_dst.copy_(copy_src)
        if not args.no_flush:
            flush()

    for i in range(Wm):
        pre_step()
        step()
        pre_step()
        two_call_step()
    torch.cuda.synchronize()
    log(f"{Wm} warmup steps done")

    def timed(fn, n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            pre_step()
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3

    # pass A (the timed K steps)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_step = timed(step, K)
    wall = time.perf_counter() - wall0
    log(f"{K} timed steps done in {wall:.3f} s wall (cache flushes included)")

    # pass B: events recorded by the library right before / after its main kernel
    evB = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for row in evB:                     # create the HIP events before use
        row[0].record(stream)
        row[1].record(stream)
    for i in range(K):
        pre_step()
        step(marks=evB[i])
    torch.cuda.synchronize()
    t_main = np.array([e[0].elapsed_time(e[1]) for e in evB]) * 1e-3
    # pass C: the same step as two calls
    t_two = timed(two_call_step, K)
    # pass D: the fused step with the rotary embedding of the new q/k fused in
    cos_np, sin_np = W.rope_table(W.MAX_CONTEXT)
    rope_cos = torch.from_numpy(cos_np).to(dev)
    rope_sin = torch.from_numpy(sin_np).to(dev)

    def rope_step():
        pa.append_decode_attention_rope(q, k_new, v_new, rope_cos, rope_sin, k_pool, v_pool,
                                        bt, lens, msl, scale=batch.scale, out=out,
                                        pages_per_split=ps, workspace=workspace, stream=stream)
    rope_step()
    t_rope = timed(rope_step, K)
    log(f"{K} breakdown, {K} two-call and {K} RoPE steps done")

    # prefill page fill of one 2048-token prompt (2 x 2 MiB moved, read + write),
    # into a scratch pool of its own so the measured cache stays untouched
    fill_rows = torch.from_numpy(np.ascontiguousarray(
        W.random_rows(np.random.default_rng(9), W.MAX_CONTEXT)).view(np.int16)).to(dev)
    fill_bt = torch.arange(W.MAX_BLOCKS, dtype=torch.int32, device=dev)
    fill_k = torch.empty((W.MAX_BLOCKS, 16, 8, 64), dtype=torch.int16, device=dev)
    fill_v = torch.empty_like(fill_k)

    def fill_step():
        pa.fill_kv(fill_rows, fill_rows, fill_bt, 0, fill_k, fill_v, stream=stream)
    fill_step()
    t_fill = timed(fill_step, K)
    fill_bytes = 2 * 2 * W.MAX_CONTEXT * 1024

    # host page allocator: one decode step of the batch (grow every sequence by
    # a token, mark the step), 16 layers, sequences crossing page boundaries
    alloc = pa.KVPool(2 * B * 16 * 128, 16, 16, W.MAX_CONTEXT)
    for rid in range(B):
        alloc.submit(rid, 1000, 1000)
    alloc.admit(capacity=B)
    for rid in range(B):
        alloc.grow(rid, 1000)
    t0 = time.perf_counter()
    n_steps = 64
    for s_i in range(n_steps):
        for rid in range(B):
            alloc.grow(rid, 1001 + s_i)
        alloc.step()
    alloc_step_us = (time.perf_counter() - t0) / n_steps * 1e6
    alloc.close()

    # the RoPE pass left rotated keys in the appended slots and its own output:
    # one more plain step restores the state the oracle recomputes
    step()
    torch.cuda.synchronize()

    # pass E: the same step over INT8 pages.  The BF16 cache is quantised on
    # the GPU page by page (every slot of every page, as one sequence over an
    # identity table), then the fused quantise-append + decode is timed.
    q8_k, q8_v, q8_s = pa.new_q8_pools(batch.num_pages, device=dev)
    npg = batch.num_pages
    ident = torch.arange(npg, dtype=torch.int32, device=dev)
    pa.fill_kv_q8(k_pool.view(npg * 16, 8, 64), v_pool.view(npg * 16, 8, 64), ident, 0,
                  q8_k, q8_v, q8_s, stream=stream)
    out_q8 = torch.empty_like(out)

    def q8_step():
        pa.append_decode_attention_q8(q, k_new, v_new, q8_k, q8_v, q8_s, bt, lens, msl,
                                      scale=batch.scale, out=out_q8, pages_per_split=ps,
                                      workspace=workspace, stream=stream)
    for _ in range(Wm):
        pre_step()
        q8_step()
    t_q8 = timed(q8_step, K)
    log(f"{K} INT8-page steps done")
    del q8_k, q8_v, q8_s

    # pass F: the same over INT4 pages (quantised on the GPU as for pass E)
    q4_k, q4_v, q4_s = pa.new_q4_pools(npg, device=dev)
    pa.fill_kv_q4(k_pool.view(npg * 16, 8, 64), v_pool.view(npg * 16, 8, 64), ident, 0,
                  q4_k, q4_v, q4_s, stream=stream)
    ps4, ns4 = pa.decode_plan_lengths_q4(batch.seq_lens, npg, max_seq_len=msl)
    out_q4 = torch.empty_like(out)
    # the INT4 plan may split where the BF16 one does not: a workspace of its own
    ws4 = torch.empty(max(pa.decode_workspace_bytes(B, msl, npg, 128, ps4), 256),
                      dtype=torch.uint8, device=dev)

    def q4_step():
        pa.append_decode_attention_q4(q, k_new, v_new, q4_k, q4_v, q4_s, bt, lens, msl,
                                      scale=batch.scale, out=out_q4, pages_per_split=ps4,
                                      workspace=ws4, stream=stream)
    for _ in range(Wm):
        pre_step()
        q4_step()
    t_q4 = timed(q4_step, K)
    log(f"{K} INT4-page steps done")
    del q4_k, q4_v, q4_s, ws4

    # diagnostic: the same step with the pages in identity order (each
    # sequence's pages consecutive in the pool)
    order = bt.reshape(-1).long()
    k_id, v_id = k_pool[order].contiguous(), v_pool[order].contiguous()
    bt_id = torch.arange(B * W.MAX_BLOCKS, dtype=torch.int32, device=dev).reshape(B, W.MAX_BLOCKS)
    out_id = torch.empty_like(out)

    def identity_step():
        pa.append_decode_attention(q, k_new, v_new, k_id, v_id, bt_id, lens, msl,
                                   scale=batch.scale, out=out_id, pages_per_split=ps,
                                   workspace=workspace, stream=stream)
    identity_step()
    t_identity = timed(identity_step, K)
    del k_id, v_id

    # what a plain streaming read of 1 GiB achieves on this device
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    pa.stream_read(flush_buf, sink, stream=stream)
    t_read = timed(lambda: pa.stream_read(flush_buf, sink, stream=stream), K)
    read_gbps = flush_buf.numel() * 4 / float(np.median(t_read)) / 1e9
    log(f"{K} identity-placement steps and {K} streaming reads done")
    by = A.step_bytes(batch.seq_lens, out_bytes=4, append=True)
    kv = by["kv"]
    by_q8 = A.step_bytes_q8(batch.seq_lens)["kv"]
    by_q4 = A.step_bytes_q4(batch.seq_lens)["kv"]
    mean_step = float(t_step.mean())
    value = kv / mean_step / 1e9
    achieved = kv / float(t_main.mean()) / 1e9

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(mean_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "paged GQA decode, 1 layer, batch 256 x 2048 tokens (1 GiB BF16 K/V), "
                        "fused append + attention",
            "global_batch": B, "seq_len": msl, "q_heads": 32, "kv_heads": 8, "head_dim": 64,
            "page_tokens": 16, "num_pages": batch.num_pages, "placement": args.placement,
            "pages_per_split": ps, "splits": ns, "out_dtype": "f32",
            "cache_flush_between_steps": not args.no_flush,
        },
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "seq_per_s_per_layer": round(B / mean_step, 1),
        "kv_gbps_main_kernel": round(kv / float(t_main.mean()) / 1e9, 2),
        "algorithmic_bytes_per_step": by,
        "all_bytes_gbps_step": round(by["total"] / mean_step / 1e9, 2),
        "times_us": {
            "step": round(mean_step * 1e6, 2),
            "step_min": round(float(t_step.min()) * 1e6, 2),
            "step_median": round(float(np.median(t_step)) * 1e6, 2),
            "wall_per_step_incl_flush": round(wall / K * 1e6, 2),
            "main_kernel": round(float(t_main.mean()) * 1e6, 2),
            "two_call_step": round(float(t_two.mean()) * 1e6, 2),
            "rope_fused_step": round(float(t_rope.mean()) * 1e6, 2),
            "prefill_fill_2048_tokens": round(float(t_fill.mean()) * 1e6, 2),
        },
        "prefill_fill_gbps": round(fill_bytes / float(t_fill.mean()) / 1e9, 1),
        "allocator_us_per_decode_step": round(alloc_step_us, 1),
        "two_call_kv_gbps": round(kv / float(t_two.mean()) / 1e9, 2),
        "achievable_read": {
            "kernel": "pa_stream_read (non-temporal 16-byte loads) over a 1 GiB buffer (median of the timed reads)",
            "gbps": round(read_gbps, 1),
            "frac_of_peak": round(read_gbps / HBM_PEAK_GBPS, 4),
            "step_value_frac_of_achievable": round(value / read_gbps, 4),
        },
        "identity_placement_step_us": round(float(t_identity.mean()) * 1e6, 2),
        "int8_pages": {
            "step_us": round(float(t_q8.mean()) * 1e6, 2),
            "step_min_us": round(float(t_q8.min()) * 1e6, 2),
            "kv_bytes": by_q8,
            "kv_gbps": round(by_q8 / float(t_q8.mean()) / 1e9, 2),
            "hbm_peak_frac": round(by_q8 / float(t_q8.mean()) / 1e9 / HBM_PEAK_GBPS, 4),
            "speedup_vs_bf16_step": round(mean_step / float(t_q8.mean()), 3),
            "seq_per_s_per_layer": round(B / float(t_q8.mean()), 1),
            "format": "int8 codes + one FP32 scale per (token, KV head) row, K and V",
            "traffic": measured_traffic(TRAFFIC_FILE_Q8, KERNEL_SOURCES_Q8),
            "kernel_source_sha": kernel_source_hash(KERNEL_SOURCES_Q8),
        },
        "int4_pages": {
            "step_us": round(float(t_q4.mean()) * 1e6, 2),
            "step_min_us": round(float(t_q4.min()) * 1e6, 2),
            "pages_per_split": ps4, "splits": ns4,
            "kv_bytes": by_q4,
            "kv_gbps": round(by_q4 / float(t_q4.mean()) / 1e9, 2),
            "hbm_peak_frac": round(by_q4 / float(t_q4.mean()) / 1e9 / HBM_PEAK_GBPS, 4),
            "speedup_vs_bf16_step": round(mean_step / float(t_q4.mean()), 3),
            "seq_per_s_per_layer": round(B / float(t_q4.mean()), 1),
            "format": "int4 codes, two per byte, + one FP32 scale per (token, KV head) row, K and V",
            "traffic": measured_traffic(TRAFFIC_FILE_Q4, KERNEL_SOURCES_Q8),
            "kernel_source_sha": kernel_source_hash(KERNEL_SOURCES_Q8),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "pa::decode_kernel (append fused)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": kv,
            "avg_launch_us": round(float(t_main.mean()) * 1e6, 2),
        },
        "kernel_source_sha": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s on one core, then "
            f"{args.cpu_seconds:.0f} s on {pool_workers} processes")
        line["cpu_baseline"] = cpu_baseline(out.cpu().numpy().astype(np.float64),
                                            args.cpu_seconds, pool, pool_workers)
        if pool is not None:
            pool.close()
            pool.join()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
