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
Pass A times the K steps with one event pair around each step, and the
library records a second pair right around its main kernel inside the same
steps (the roofline figure); pass C times the two-call form; pass D the
fused step with RoPE; pass E the fused step over INT8 pages and pass F over
INT4 pages (the BF16 cache quantised on the GPU first).  Two diagnostics
follow: the same step with the pages in identity order, and a plain
streaming read of 1 GiB (the achievable read bandwidth, beside the published
peak).  The flush is outside every event pair.

Then every other configuration (1: one 37-token sequence; 2: batch 8 of
uniform lengths; 3: the 16-layer step of batch 64; 5: batch 512 of clipped
Zipf lengths) is measured the same way, its fused step under each candidate
launch (the default plan, the host-lengths plan, the work list, the balanced
launch over a host plan), the fastest
reported, with every output compared against the oracle.  The oracle runs on
one core and on a pool of worker processes forked before the GPU is
initialised, on every configuration.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
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
BALANCED_SOURCES = [os.path.join(_CSRC, n) for n in _DEVICE + ("pa_balance_plan.h",
                                                             "pa_decode_balanced.hip")]
STREAM_SOURCES = [os.path.join(_CSRC, n) for n in _DEVICE + ("pa_measure.hip",)]
# (wavefronts per KV head, LDS ring slots) of the decode kernels on the 256 x 2048
# batch: BF16 pages one wavefront per KV head and one slot, INT8 pages one and
# two; INT4 pages two wavefronts per KV head (one 128-page split per sequence)
# and three slots
STREAM_SHAPES = {"bf16": (1, 1), "int8": (1, 2), "int4": (2, 3)}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash(sources=None) -> str:
    """sha256[:16] of the kernel sources' code: comments and blank lines are left
    out, so that a summary keyed to it survives an edit of the prose alone."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            code = _COMMENTS.sub("", f.read())
        h.update("\n".join(l.rstrip() for l in code.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def source_hashes() -> dict:
    """sha256[:16] of each kernel family's sources, printed ahead of the tables of
    the sweep, the placement probe and the one-configuration runs, so that a
    summary can tell which sources it describes."""
    return {"grid_bf16": kernel_source_hash(KERNEL_SOURCES),
            "grid_quantised": kernel_source_hash(KERNEL_SOURCES_Q8),
            "balanced": kernel_source_hash(BALANCED_SOURCES),
            "page_stream": kernel_source_hash(STREAM_SOURCES)}


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


TRACE_FILE = os.path.join(ROOT, "profiles", "decode_kernel_trace_b256_l2048.json")


def rocprof_kernel_time(path: str = TRACE_FILE):
    """The main kernel's average duration from the committed rocprofv3 kernel
    trace of this workload, and the roofline fraction it gives; None when
    absent or when the kernel has changed since."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    us = float(t["avg_us"])
    gbps = t["algorithmic_kv_bytes"] / us / 1e3
    return {"avg_us": us, "achieved": round(gbps, 2), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "calls": t.get("calls"), "source": os.path.relpath(path, ROOT)}


# host inputs of every measured configuration, set before the pool forks:
# {config: [(batch, k_ref, v_ref) per layer]}, k_ref/v_ref the oracle's pools
# after the append (the workers inherit them and never touch the GPU)
_STATES = {}
CONFIGS = (1, 2, 3, 4, 5)


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def config_layers(ci: int, placement: str = "random"):
    """Host inputs of configuration ``ci`` with the append: one batch per layer
    (16 for configuration 3, one pool region each)."""
    import workloads as W
    if ci == 3:
        return [W.make_workload(3, layer=layer, placement=placement, append=True)
                for layer in range(W.NUM_LAYERS_W3)]
    return [W.make_workload(ci, placement=placement, append=True)]


def page_stream_entry(fmt: str, nbytes: int, t_stream, t_step) -> dict:
    """One page format's stream time beside its fused step's (both medians)."""
    import numpy as np
    wph, ring = STREAM_SHAPES[fmt]
    us, step_us = float(np.median(t_stream)) * 1e6, float(np.median(t_step)) * 1e6
    return {"waves_per_head": wph, "ring": ring, "us": round(us, 2),
            "gbps": round(nbytes / us / 1e3, 1),
            "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4),
            "step_median_us": round(step_us, 2),
            "step_over_stream": round(step_us / us, 4)}


def prepare_states(configs, placement: str, headline=None):
    """Inputs and the oracle's appended pools of each configuration (host only)."""
    import oracle
    for ci in configs:
        t0 = time.perf_counter()
        layers = [headline] if (ci == 4 and headline is not None) else config_layers(ci, placement)
        st = []
        for w in layers:
            k_ref, v_ref = oracle.append_kv(w.k_pool, w.v_pool, w.k_new, w.v_new,
                                            w.block_tables, w.seq_lens)
            st.append((w, k_ref, v_ref))
        _STATES[ci] = st
        log(f"config {ci}: {len(st)} layer(s) x {st[0][0].batch} sequences generated in "
            f"{time.perf_counter() - t0:.1f} s")


def _items(ci):
    """(layer, sequence) pairs of configuration ``ci``, layer by layer."""
    return [(li, b) for li, (w, _, _) in enumerate(_STATES[ci]) for b in range(w.batch)]


def _oracle_decodes(ci: int, first: int, stride: int, seconds: float, gpu_outs=None):
    """Decode items first, first+stride, ... (cycling) with the oracle for ``seconds``.

    Returns (items done, seconds, tokens, max-abs against ``gpu_outs`` [layer][B][32][64]).
    """
    import numpy as np
    import oracle
    items = _items(ci)
    done, tokens, worst, t0 = 0, 0, 0.0, time.perf_counter()
    while True:
        li, b = items[(first + stride * done) % len(items)]
        w, k_ref, v_ref = _STATES[ci][li]
        ref = oracle.decode_attention(w.q, k_ref, v_ref, w.block_tables, w.seq_lens, w.scale,
                                      sequences=[b])
        if gpu_outs is not None:
            worst = max(worst, float(np.max(np.abs(ref[b] - gpu_outs[li][b]))))
        done += 1
        tokens += int(w.seq_lens[b])
        if time.perf_counter() - t0 >= seconds and done >= 2:
            break
    return done, time.perf_counter() - t0, tokens, worst


def _pool_leg(args):
    ci, first, stride, seconds = args
    done, dt, tokens, _ = _oracle_decodes(ci, first, stride, seconds)
    return done, dt, tokens


def fork_pool(pool_workers: int):
    """The oracle's worker processes, forked before the GPU is first touched."""
    import multiprocessing as mp
    if pool_workers <= 1:
        return None
    return mp.get_context("fork").Pool(pool_workers, initializer=_blas_one_thread)


def oracle_rates(ci: int, seconds: float, pool=None, pool_workers: int = 0, gpu_outs=None):
    """The oracle, as it stands, on configuration ``ci``: one core, then the process pool."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = contextlib.nullcontext()
    with limit:
        done, dt, tokens, worst = _oracle_decodes(ci, 0, 1, seconds, gpu_outs)
    kv = tokens * 2048
    res = {
        "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{done} sequence decodes cycling over the {len(_items(ci))} (layer, sequence) "
                   f"pairs ({tokens} tokens, {kv / 2**20:.0f} MiB of K/V), float64 NumPy, "
                   f"1 BLAS thread, {dt:.1f} s"),
        "seq_per_s": round(done / dt, 3),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": 1,
    }
    if gpu_outs is not None:
        res["max_abs_vs_gpu_on_sample"] = worst
    if pool is not None:
        t0 = time.perf_counter()
        legs = pool.map(_pool_leg, [(ci, w, pool_workers, seconds) for w in range(pool_workers)])
        wall = time.perf_counter() - t0
        n = sum(d for d, _, _ in legs)
        ptok = sum(t for _, _, t in legs)
        res["pool"] = {
            "value": round(ptok * 2048 / wall / 1e9, 4), "unit": "GB/s", "cores": pool_workers,
            "sample": (f"{n} sequence decodes over {pool_workers} worker processes "
                       f"(1 BLAS thread each), {wall:.1f} s wall"),
            "seq_per_s": round(n / wall, 3),
        }
    return res


def oracle_refs(ci: int):
    """The oracle's output of every sequence of every layer of configuration ``ci``."""
    import oracle
    return [oracle.decode_attention(w.q, k, v, w.block_tables, w.seq_lens, w.scale)
            for w, k, v in _STATES[ci]]


def parity(gpu_outs, refs):
    """(max-abs, max-rel with denominator max(|ref|, 1e-2)) over every element."""
    import numpy as np
    err = max(float(np.max(np.abs(g - r))) for g, r in zip(gpu_outs, refs))
    rel = max(float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-2)))
              for g, r in zip(gpu_outs, refs))
    return err, rel


def measure_config(ci: int, args, stream, dev, flush, refs):
    """Every candidate launch of configuration ``ci``'s fused step (all its
    layers back to back), cold caches; the fastest is the configuration's figure."""
    import numpy as np
    import torch

    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    states = _STATES[ci]
    w0 = states[0][0]
    B, npg, msl = w0.batch, w0.num_pages, w0.max_seq_len
    layers = [dict(q=up16(w.q), kp=up16(w.k_pool), vp=up16(w.v_pool), kn=up16(w.k_new),
                   vn=up16(w.v_new), bt=torch.from_numpy(w.block_tables).to(dev),
                   lens=torch.from_numpy(w.seq_lens).to(dev),
                   out=torch.empty((B, 32, 64), dtype=torch.float32, device=dev))
              for w, _, _ in states]
    kv = sum(A.step_bytes(w.seq_lens, append=True)["kv"] for w, _, _ in states)
    cands = [("grid, default plan (pages_per_split=0)", 0, None)]
    ps_l, _ = pa.decode_plan_lengths(w0.seq_lens, npg, max_seq_len=msl)
    cands.append(("grid, host-lengths plan", ps_l, None))
    if B > 1:
        wl, wps, _ = pa.decode_worklist(w0.seq_lens, npg, max_seq_len=msl)
        cands.append(("work list", wps, torch.from_numpy(wl).to(dev)))
    for h in (8, 2, 1):
        try:
            plan = pa.balance_plan(w0.seq_lens, npg, max_seq_len=msl, heads_together=h,
                                   device=dev)
        except RuntimeError:
            continue                       # this batch cannot be planned with such lanes
        cands.append((f"balanced, {h} KV head{'s' if h > 1 else ''} per lane", 0, plan))
    # host time of the planning call each launch needs for this batch of
    # lengths (a serving loop makes it once per step): median of 20 calls
    def host_us(fn):
        t = []
        for _ in range(20):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return round(float(np.median(t)) * 1e6, 1)
    plan_us = {"grid, host-lengths plan": host_us(
        lambda: pa.decode_plan_lengths(w0.seq_lens, npg, max_seq_len=msl))}
    if B > 1:
        plan_us["work list"] = host_us(
            lambda: pa.decode_worklist(w0.seq_lens, npg, max_seq_len=msl))
    for name, _, work in cands:
        if isinstance(work, pa.BalancedPlan):
            h = int(name.split(", ")[1].split(" ")[0])
            plan_us[name] = host_us(lambda h=h: pa.balance_plan(
                w0.seq_lens, npg, max_seq_len=msl, heads_together=h, host_only=True))
    need = max(pa.decode_workspace_bytes(B, msl, npg, 128, ps) for _, ps, _ in cands)
    workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def run(ps, work):
        for L in layers:
            if isinstance(work, pa.BalancedPlan):
                pa.decode_balanced(L["q"], L["kp"], L["vp"], L["bt"], L["lens"], msl, work,
                                   k_new=L["kn"], v_new=L["vn"], scale=w0.scale, out=L["out"],
                                   stream=stream)
            elif work is None:
                pa.append_decode_attention(L["q"], L["kn"], L["vn"], L["kp"], L["vp"], L["bt"],
                                           L["lens"], msl, scale=w0.scale, out=L["out"],
                                           pages_per_split=ps, workspace=workspace, stream=stream)
            else:
                pa.append_decode_attention_worklist(
                    L["q"], L["kn"], L["vn"], L["kp"], L["vp"], L["bt"], L["lens"], msl, work,
                    ps, scale=w0.scale, out=L["out"], workspace=workspace, stream=stream)

    res, best = {}, None
    for name, ps, work in cands:
        for _ in range(max(args.warmup, 1)):
            flush()
            run(ps, work)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in evs:
            flush()
            e[0].record(stream)
            run(ps, work)
            e[1].record(stream)
        torch.cuda.synchronize()
        t = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        outs = [L["out"].cpu().numpy().astype(np.float64) for L in layers]
        err, rel = parity(outs, refs) if refs is not None else (None, None)
        res[name] = {"pages_per_split": int(ps), "step_us": round(float(t.mean()) * 1e6, 2),
                     "step_median_us": round(float(np.median(t)) * 1e6, 2),
                     "step_min_us": round(float(t.min()) * 1e6, 2),
                     "kv_gbps": round(kv / float(t.mean()) / 1e9, 1),
                     "plan_host_us": plan_us.get(name, 0.0),
                     "max_abs_vs_oracle": err, "max_rel_vs_oracle": rel}
        if best is None or t.mean() < best[1]:
            best = (name, float(t.mean()), outs)
    name, t_best, outs = best
    nl = len(layers)
    line = {
        "workload": states[0][0].recipe.get("workload", ""), "layers": nl, "batch": B,
        "launch": name, "pages_per_split": res[name]["pages_per_split"],
        "plan_host_us": res[name]["plan_host_us"],
        "step_us": round(t_best * 1e6, 2), "step_median_us": res[name]["step_median_us"],
        "step_min_us": res[name]["step_min_us"], "per_layer_us": round(t_best / nl * 1e6, 2),
        "kv_bytes": int(kv), "kv_gbps": round(kv / t_best / 1e9, 1),
        "hbm_peak_frac": round(kv / t_best / 1e9 / HBM_PEAK_GBPS, 4),
        "seq_per_s_per_layer": round(int(np.count_nonzero(w0.seq_lens)) * nl / t_best, 1),
        "max_abs_vs_oracle": res[name]["max_abs_vs_oracle"],
        "max_rel_vs_oracle": res[name]["max_rel_vs_oracle"],
        "launches": res,
    }
    del layers, workspace
    torch.cuda.empty_cache()
    return line, outs


def run_sweep(args) -> int:
    """Every workload's fused append + attention step (one layer; workload 3 is its
    first layer), cold caches, medians of ``--steps`` event-timed steps."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    print(json.dumps({"kernel_sources": source_hashes()}), flush=True)
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

    for wi in (1, 2, 3, 4, 5, 6):
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
            for h in (8, 1):
                try:
                    plan = pa.balance_plan(w.seq_lens, npg, max_seq_len=msl, heads_together=h,
                                           device=dev)
                except RuntimeError:
                    continue
                cases.append((f"balanced, {h} KV head{'s' if h > 1 else ''} per lane", 0,
                              plan.groups,
                              lambda plan=plan, kpool=kpool, vpool=vpool, scales=scales:
                              pa.decode_balanced(q, kpool, vpool, bt, lens, msl, plan,
                                                 k_new=kn, v_new=vn, kv_scales=scales,
                                                 scale=w.scale, out=out, stream=stream)))
            for launch, cps, units, fn in cases:
                t = timed(fn, args.steps)
                unit_key = ("items" if launch == "work list" else
                            "work_groups" if launch.startswith("balanced") else "splits")
                print(json.dumps({
                    "workload": wi, "desc": W.WORKLOADS[wi], "pages": fmt,
                    "launch": launch, "pages_per_split": int(cps),
                    unit_key: int(units),
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


def parse_configs(text: str):
    """Configurations of ``--configs`` (sorted, unique), or None if one is not 1, 2, 3 or 5."""
    try:
        cs = sorted(set(int(c) for c in text.split(",") if c.strip()))
    except ValueError:
        return None
    return None if any(c not in CONFIGS or c == 4 for c in cs) else cs


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
    ap.add_argument("--configs", default="1,2,3,5",
                    help="configurations measured beside the headline (comma list of 1-5; "
                         "'' for none): each one's fused step, its oracle rates and its "
                         "max-abs over every output")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="oracle time per configuration, one core and then the pool")
    ap.add_argument("--only-config", type=int, default=0,
                    help="measure this one configuration's candidate launches only (no "
                         "headline passes, no oracle): for profiling runs")
    ap.add_argument("--placement-probe", action="store_true",
                    help="instead of the bench line: the decode kernel on batch 256 x 2048 with "
                         "the same logical cache under several page placements (identity, "
                         "per-sequence regions, random chunks of 4..64 pages, one random "
                         "permutation), interleaved, cold caches; one JSON line per placement")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: time the fused step of every workload "
                         "(1-6; 6 is the truncated reading of workload 5's Zipf lengths), BF16, "
                         "INT8 and INT4 pages, under every launch; one JSON line per case")
    ap.add_argument("--page-stream", action="store_true",
                    help="instead of the bench line: the decode kernels' page reads alone "
                         "(pa_page_stream) on batch 256 x 2048 for every page format, "
                         "wavefronts per KV head and ring depth, beside each format's decode "
                         "kernel, interleaved, cold caches; one JSON line per case")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the bench line: the balanced launch with per-wavefront "
                         "real-time stamps (pa_decode_balanced_timeline) on workloads 3, 4 and 5, "
                         "beside the plain launch, interleaved, cold caches; one JSON line per "
                         "case with the phases of each launch")
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
    if args.placement_probe:
        return run_placement_probe(args)
    if args.page_stream:
        return run_page_stream(args)
    if args.timeline:
        return run_timeline(args)
    if args.only_config:
        if args.only_config not in CONFIGS:
            print("--only-config takes 1..5", file=sys.stderr)
            return 2
        return run_one_config(args)

    others = parse_configs(args.configs)
    if others is None:
        print("--configs takes configurations 1, 2, 3 and 5 (4 is the headline)", file=sys.stderr)
        return 2
    t0 = time.perf_counter()
    batch = W.make_workload(4, placement=args.placement, append=True)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s "
        f"({batch.batch} sequences, {batch.num_pages} pages)")
    prepare_states([4] + others, args.placement, headline=batch)
    pool, pool_workers = None, 0
    if not args.no_cpu_baseline:
        pool_workers = args.cpu_workers or min(len(os.sched_getaffinity(0)), 16)
        pool = fork_pool(pool_workers)

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

    # pass A: the timed K steps, each bracketed by an event pair.  When the
    # plan is one launch (one split per sequence, the append fused) the step
    # is the main kernel and the same pair times it; otherwise pass B repeats
    # the steps with the library also recording a pair right around its main
    # kernel, inside the same steps, and reports those steps' times beside it.
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_step = timed(step, K)
    wall = time.perf_counter() - wall0
    if ns == 1:
        t_main, t_step_b = t_step, t_step
        main_timing = ("the step is one launch of the main kernel: its event pair (recorded on "
                       "the launch stream, dispatch included) times both")
    else:
        evB = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for row in evB:                 # create the HIP events before use
            for e in row:
                e.record(stream)
        for i in range(K):
            pre_step()
            evB[i][0].record(stream)
            step(marks=(evB[i][1], evB[i][2]))
            evB[i][3].record(stream)
        torch.cuda.synchronize()
        t_step_b = np.array([e[0].elapsed_time(e[3]) for e in evB]) * 1e-3
        t_main = np.array([e[1].elapsed_time(e[2]) for e in evB]) * 1e-3
        main_timing = ("events recorded by the library around the main kernel inside the "
                       "steps of pass B (step_with_kernel_events_us)")
    log(f"{K} timed steps done in {wall:.3f} s wall (cache flushes included)")
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
    # the same pages read by the decode kernel's loads alone (no arithmetic)
    ps_sink = torch.empty((B, 16), dtype=torch.int32, device=dev)

    def page_stream_fn(kp, vp, sp, fmt):
        wph, ring = STREAM_SHAPES[fmt]
        return lambda: pa.page_stream(kp, vp, sp, bt, lens, wph, ring, sink=ps_sink, stream=stream)
    q8_stream = page_stream_fn(q8_k, q8_v, q8_s, "int8")
    q8_stream()
    t_q8_stream = timed(q8_stream, K)
    log(f"{K} INT8-page steps and page streams done")
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
    q4_stream = page_stream_fn(q4_k, q4_v, q4_s, "int4")
    q4_stream()
    t_q4_stream = timed(q4_stream, K)
    log(f"{K} INT4-page steps and page streams done")
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

    bf_stream = page_stream_fn(k_pool, v_pool, None, "bf16")
    bf_stream()
    t_bf_stream = timed(bf_stream, K)

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
        "page_stream": {
            "kernel": "pa_page_stream: each format's pages requested with the decode kernel's "
                      "own loads, ring and waits and read back from LDS, no attention "
                      "arithmetic (medians of the timed launches, cold caches)",
            **{fmt: page_stream_entry(fmt, by_b, t_s, t_k)
               for fmt, by_b, t_s, t_k in (("bf16", kv, t_bf_stream, t_step),
                                           ("int8", by_q8, t_q8_stream, t_q8),
                                           ("int4", by_q4, t_q4_stream, t_q4))},
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
            "timing": main_timing,
            "step_with_kernel_events_us": round(float(t_step_b.mean()) * 1e6, 2),
            "rocprof": rocprof_kernel_time(),
        },
        "kernel_source_sha": kernel_source_hash(),
    }
    out_host = out.cpu().numpy().astype(np.float64)
    del out_id, q, k_pool, v_pool, k_new, v_new, workspace
    torch.cuda.empty_cache()

    # every configuration: the fastest candidate launch of its fused step, its
    # parity over every output, the oracle beside it
    configs = {}
    refs4 = oracle_refs(4)
    err4, rel4 = parity([out_host], refs4)
    configs["4"] = {
        "workload": W.WORKLOADS[4], "layers": 1, "batch": B, "launch": "grid, default plan "
        "(pages_per_split=0)", "pages_per_split": ps, "step_us": round(mean_step * 1e6, 2),
        "step_median_us": round(float(np.median(t_step)) * 1e6, 2),
        "step_min_us": round(float(t_step.min()) * 1e6, 2),
        "per_layer_us": round(mean_step * 1e6, 2), "kv_bytes": int(kv),
        "kv_gbps": round(value, 1), "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "seq_per_s_per_layer": round(B / mean_step, 1), "max_abs_vs_oracle": err4,
        "max_rel_vs_oracle": rel4, "note": "the headline line's own figures"}
    for ci in others:
        t0 = time.perf_counter()
        refs = oracle_refs(ci)
        configs[str(ci)], _ = measure_config(ci, args, stream, dev, flush, refs)
        c = configs[str(ci)]
        log(f"config {ci}: {c['launch']}, {c['per_layer_us']} us per layer, {c['kv_gbps']} GB/s, "
            f"max-abs {c['max_abs_vs_oracle']:.2e} ({time.perf_counter() - t0:.1f} s)")
    line["configs"] = configs

    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s on one core, then "
            f"{args.cpu_seconds:.0f} s on {pool_workers} processes")
        line["cpu_baseline"] = oracle_rates(4, args.cpu_seconds, pool, pool_workers,
                                            gpu_outs=[out_host])
        for ci in others:
            configs[str(ci)]["oracle"] = oracle_rates(ci, args.config_cpu_seconds, pool,
                                                      pool_workers)
        configs["4"]["oracle"] = {k: line["cpu_baseline"][k] for k in
                                  ("value", "unit", "cores", "seq_per_s", "pool")
                                  if k in line["cpu_baseline"]}
        log(f"oracle rates of configurations {others} done")
        if pool is not None:
            pool.close()
            pool.join()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


def placement_tables(B: int, per: int, scheme: str, seed: int = 77):
    """Block tables [B][per] over a pool of exactly B * per pages for a placement scheme:
    ``identity`` (sequence b on pages b*per ..), ``region`` (the same pages, shuffled within
    the sequence), ``chunksN`` (random N-page chunks of the pool, pages shuffled within each
    chunk), ``random`` (one random permutation of the pool)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    n = B * per
    if scheme == "identity":
        flat = np.arange(n)
    elif scheme == "region":
        flat = np.concatenate([b * per + rng.permutation(per) for b in range(B)])
    elif scheme.startswith("chunks"):
        c = int(scheme[6:])
        chunks = rng.permutation(n // c)
        flat = np.concatenate([k * c + rng.permutation(c) for k in chunks])
    elif scheme == "random":
        flat = rng.permutation(n)
    else:
        raise ValueError(scheme)
    return flat.reshape(B, per).astype(np.int32)


def run_placement_probe(args) -> int:
    """The decode kernel over the 256 x 2048 cache under several page placements."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    print(json.dumps({"kernel_sources": source_hashes()}), flush=True)
    w = W.make_workload(4, append=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)
    flush_out = torch.empty((), dtype=torch.int32, device=dev)
    B, per = w.batch, W.MAX_BLOCKS
    kp = torch.from_numpy(w.k_pool.view(np.int16)).to(dev)
    vp = torch.from_numpy(w.v_pool.view(np.int16)).to(dev)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    old = torch.from_numpy(w.block_tables[:, :per].reshape(-1).astype(np.int64)).to(dev)
    schemes = ["identity", "region", "chunks4", "chunks16", "chunks32", "chunks64", "random"]
    cases = {}
    for sch in schemes:
        bt = placement_tables(B, per, sch)
        new = torch.from_numpy(bt.reshape(-1).astype(np.int64)).to(dev)
        k2, v2 = torch.empty_like(kp), torch.empty_like(vp)
        k2[new] = kp[old]                     # the same logical cache at the new places
        v2[new] = vp[old]
        cases[sch] = (k2, v2, torch.from_numpy(bt).to(dev),
                      torch.empty((B, 32, 64), dtype=torch.float32, device=dev))
    del kp, vp
    ref = None
    times = {s: [] for s in schemes}
    for it in range(args.warmup + args.steps):
        for sch in schemes:                    # interleaved: drift hits every placement alike
            k2, v2, bt, out = cases[sch]
            torch.amax(flush_buf, dim=None, out=flush_out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.decode_attention(q, k2, v2, bt, lens, w.max_seq_len, scale=w.scale, out=out,
                                stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if it >= args.warmup:
                times[sch].append(e0.elapsed_time(e1) * 1e3)
    kv = A.step_bytes(w.seq_lens)["kv"]
    for sch in schemes:
        out = cases[sch][3].cpu().numpy()
        ref = out if ref is None else ref
        t = float(np.median(times[sch]))
        print(json.dumps({"placement": sch, "decode_us_median": round(t, 2),
                          "decode_us_min": round(float(np.min(times[sch])), 2),
                          "kv_gbps": round(kv / t / 1e3, 1), "steps": args.steps,
                          "same_output_as_identity": bool(np.array_equal(out, ref))}), flush=True)
    return 0


def run_page_stream(args) -> int:
    """pa_page_stream on the 256 x 2048 cache for every page format, wavefronts per
    KV head and ring depth, beside each format's decode kernel; interleaved,
    cold caches; one JSON line per case."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_decode_07_amd import accounting as A
    from paged_kv_decode_07_amd import binding as pa

    print(json.dumps({"kernel_sources": source_hashes()}), flush=True)
    w = W.make_workload(4, append=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)
    flush_out = torch.empty((), dtype=torch.int32, device=dev)
    B, npg = w.batch, w.num_pages
    kp = torch.from_numpy(w.k_pool.view(np.int16)).to(dev)
    vp = torch.from_numpy(w.v_pool.view(np.int16)).to(dev)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    ident = torch.arange(npg, dtype=torch.int32, device=dev)
    pools = {"bf16": (kp, vp, None)}
    for fmt, new, fill in (("int8", pa.new_q8_pools, pa.fill_kv_q8),
                           ("int4", pa.new_q4_pools, pa.fill_kv_q4)):
        kc, vc, sc = new(npg, device=dev)
        fill(kp.view(npg * 16, 8, 64), vp.view(npg * 16, 8, 64), ident, 0, kc, vc, sc,
             stream=stream)
        pools[fmt] = (kc, vc, sc)
    nbytes = {"bf16": A.step_bytes(w.seq_lens)["kv"], "int8": A.step_bytes_q8(w.seq_lens)["kv"],
              "int4": A.step_bytes_q4(w.seq_lens)["kv"]}
    sink = torch.empty((B, 16), dtype=torch.int32, device=dev)
    out = torch.empty((B, 32, 64), dtype=torch.float32, device=dev)
    cases = {}
    for fmt, (kc, vc, sc) in pools.items():
        if fmt == "bf16":
            cases[(fmt, "decode kernel", 0, 0)] = lambda: pa.decode_attention(
                q, kp, vp, bt, lens, w.max_seq_len, scale=w.scale, out=out, stream=stream)
        else:
            cases[(fmt, "decode kernel", 0, 0)] = (
                lambda kc=kc, vc=vc, sc=sc, nb=8 if fmt == "int8" else 4: pa.decode_attention_q8(
                    q, kc, vc, sc, bt, lens, w.max_seq_len, scale=w.scale, out=out,
                    stream=stream, nbits=nb))
        for wph in (1, 2):
            for ring in (1, 2, 3):
                if (fmt, wph, ring) == ("bf16", 2, 3):
                    continue                      # 192 KiB of LDS ring
                cases[(fmt, "page stream", wph, ring)] = (
                    lambda kc=kc, vc=vc, sc=sc, wph=wph, ring=ring: pa.page_stream(
                        kc, vc, sc, bt, lens, wph, ring, sink=sink, stream=stream))
    times = {c: [] for c in cases}
    for it in range(args.warmup + args.steps):
        for c, fn in cases.items():               # interleaved: drift hits every case alike
            torch.amax(flush_buf, dim=None, out=flush_out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if it >= args.warmup:
                times[c].append(e0.elapsed_time(e1) * 1e3)
    for (fmt, what, wph, ring), t in times.items():
        med = float(np.median(t))
        line = {"format": fmt, "case": what, "us_median": round(med, 2),
                "us_min": round(float(np.min(t)), 2), "gbps": round(nbytes[fmt] / med / 1e3, 1),
                "frac_of_peak": round(nbytes[fmt] / med / 1e3 / HBM_PEAK_GBPS, 4),
                "steps": args.steps}
        if what == "page stream":
            line.update({"waves_per_head": wph, "ring": ring,
                         "decode_kernel_shape": STREAM_SHAPES[fmt] == (wph, ring)})
        print(json.dumps(line), flush=True)
    return 0


TIMELINE_CASES = ((3, 1), (4, 8), (5, 8))     # (workload, KV heads per lane)


def timeline_phases(stamps, khz: float) -> dict:
    """Phases of one launch from its timeline stamps (int64 [groups][8][8]):
    medians over wavefronts, and the work-groups' end times."""
    import numpy as np
    us = 1e3 / khz
    t = stamps[..., :7].astype(np.int64)
    w7 = stamps[..., 7].astype(np.int64)
    pages = (w7 >> 48) & 0xFFFF
    xcc = ((w7 >> 32) & 0xFFFF)[:, 0]
    base = t[..., 0].min()
    busy = pages > 0
    runs = pages >= 2
    wg_end = (t[..., 6].max(axis=1) - base) * us
    per_page = (t[..., 4] - t[..., 3])[runs] * us / (pages[runs] - 1)
    out = {
        "span_us": float((t[..., 6].max() - base) * us),
        "dispatch_us": float((t[..., 0].max() - base) * us),
        "descriptor_us": float(np.median(t[..., 1] - t[..., 0]) * us),
        "metadata_us": float(np.median(t[..., 2] - t[..., 1]) * us),
        "first_page_us": float(np.median((t[..., 3] - t[..., 2])[busy]) * us),
        "first_page_at_us": float(np.median((t[..., 3] - base)[busy]) * us),
        "stream_us": float(np.median((t[..., 4] - t[..., 3])[busy]) * us),
        "us_per_page": float(np.median(per_page)) if per_page.size else None,
        "tail_us": float(np.median(t[..., 6] - t[..., 4]) * us),
        "wg_end_us": wg_end,
        "xcc": xcc,
        "per_page_by_wg": np.array([np.median((t[g, :, 4] - t[g, :, 3])[runs[g]] * us /
                                              (pages[g][runs[g]] - 1)) if runs[g].any() else np.nan
                                    for g in range(t.shape[0])]),
        "base": int(base), "end": int(t[..., 6].max()),
        "pages": pages,
    }
    return out


def run_timeline(args) -> int:
    """The balanced launch with per-wavefront timeline stamps on workloads 3 (16
    layers, one KV head per lane), 4 and 5 (8 heads per lane): where each
    launch's time goes.  One JSON line per case."""
    import numpy as np
    import torch
    from paged_kv_decode_07_amd import binding as pa

    print(json.dumps({"kernel_sources": source_hashes()}), flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    khz = pa.wall_clock_khz()
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)
    flush_out = torch.empty((), dtype=torch.int32, device=dev)

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    for ci, h in TIMELINE_CASES:
        hosts = config_layers(ci, args.placement)
        w0 = hosts[0]
        B, msl = w0.batch, w0.max_seq_len
        layers = [dict(q=up16(w.q), kp=up16(w.k_pool), vp=up16(w.v_pool), kn=up16(w.k_new),
                       vn=up16(w.v_new), bt=torch.from_numpy(w.block_tables).to(dev),
                       lens=torch.from_numpy(w.seq_lens).to(dev),
                       out=torch.empty((B, 32, 64), dtype=torch.float32, device=dev))
                  for w in hosts]
        plan = pa.balance_plan(w0.seq_lens, w0.num_pages, max_seq_len=msl, heads_together=h,
                               device=dev)
        stamps = [torch.zeros((plan.groups, 8, 8), dtype=torch.int64, device=dev) for _ in layers]

        def step(timed):
            for L, st in zip(layers, stamps):
                if timed:
                    pa.decode_balanced_timeline(L["q"], L["kp"], L["vp"], L["bt"], L["lens"], msl,
                                                plan, k_new=L["kn"], v_new=L["vn"], scale=w0.scale,
                                                out=L["out"], stamps=st, stream=stream)
                else:
                    pa.decode_balanced(L["q"], L["kp"], L["vp"], L["bt"], L["lens"], msl, plan,
                                       k_new=L["kn"], v_new=L["vn"], scale=w0.scale,
                                       out=L["out"], stream=stream)
        t_tl, t_plain, phases = [], [], []
        for it in range(args.warmup + args.steps):
            for timed in (True, False):            # interleaved: drift hits both alike
                torch.amax(flush_buf, dim=None, out=flush_out)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step(timed)
                e1.record(stream)
                torch.cuda.synchronize()
                if it < args.warmup:
                    continue
                (t_tl if timed else t_plain).append(e0.elapsed_time(e1) * 1e3)
                if timed:
                    phases.append([timeline_phases(st.cpu().numpy(), khz) for st in stamps])
        nl = len(layers)
        us = 1e3 / khz
        keys = ("span_us", "dispatch_us", "descriptor_us", "metadata_us", "first_page_us",
                "first_page_at_us", "stream_us", "us_per_page", "tail_us")
        med = {k: round(float(np.median([p[k] for ps in phases for p in ps if p[k] is not None])),
                        3) for k in keys}
        gaps = [(ps[l]["base"] - ps[l - 1]["end"]) * us for ps in phases for l in range(1, nl)]
        ends = np.concatenate([p["wg_end_us"] for ps in phases for p in ps])
        # per die: the work-groups' end times and per-page times, over every launch
        xcc = np.concatenate([p["xcc"] for ps in phases for p in ps])
        ppg = np.concatenate([p["per_page_by_wg"] for ps in phases for p in ps])
        by_xcc = {str(int(x)): {"wg_end_median_us": round(float(np.median(ends[xcc == x])), 2),
                                "us_per_page": round(float(np.nanmedian(ppg[xcc == x])), 3),
                                "work_groups": int((xcc == x).sum()) // len(phases)}
                  for x in np.unique(xcc)}
        # stamped time over event time: spans and gaps of the step against the events
        cover = [(ps[-1]["end"] - ps[0]["base"]) * us / t for ps, t in zip(phases, t_tl)]
        pg = phases[0][0]["pages"]
        line = {
            "case": f"workload {ci}, balanced, {h} KV head{'s' if h > 1 else ''} per lane",
            "workload": ci, "layers": nl, "batch": B, "heads_together": h,
            "groups": plan.groups, "steps": args.steps, "warmup": args.warmup,
            "clock_khz": khz,
            "step_us_timeline": round(float(np.median(t_tl)), 2),
            "step_us_plain": round(float(np.median(t_plain)), 2),
            "per_layer_us_plain": round(float(np.median(t_plain)) / nl, 2),
            "gap_us": round(float(np.median(gaps)), 3) if gaps else None,
            **med,
            "wg_end_us": {q: round(float(np.percentile(ends, v)), 2)
                          for q, v in (("min", 0), ("p10", 10), ("p50", 50), ("p90", 90),
                                       ("max", 100))},
            "by_xcc": by_xcc,
            "pages_per_wave": {"min": int(pg.min()), "median": float(np.median(pg)),
                               "max": int(pg.max())},
            "stamped_over_event": round(float(np.median(cover)), 4),
        }
        print(json.dumps(line), flush=True)
        del layers, stamps
        torch.cuda.empty_cache()
    return 0


def run_one_config(args) -> int:
    """Only configuration ``--only-config``'s candidate launches (no oracle, no
    headline passes): one JSON line; for profiling runs."""
    import torch
    from paged_kv_decode_07_amd import binding as pa
    ci = args.only_config
    prepare_states([ci], args.placement)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(2**28, dtype=torch.int32, device=dev)
    flush_out = torch.empty((), dtype=torch.int32, device=dev)

    def flush():
        if not args.no_flush:
            torch.amax(flush_buf, dim=None, out=flush_out)
    if args.calibration_copy:
        # one 256 MiB device copy: the known-size reference for byte counters
        src = torch.ones(2**26, dtype=torch.int32, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    line, _ = measure_config(ci, args, stream, dev, flush, None)
    print(json.dumps({"config": ci, **line, "kernel_sources": source_hashes()}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
