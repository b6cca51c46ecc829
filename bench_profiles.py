"""Summaries under profiles/ from rocprofv3 runs of bench.py.

Modes (the first two read rocprofv3 output directories, ``-f csv -d DIR``):

  python bench_profiles.py headline --line FILE --trace DIR --fetch DIR --write DIR [--util DIR]
      runs of ``bench.py --no-cpu-baseline --configs ''`` (the batch 256 x 2048
      line): the kernel trace (profiles/decode_kernel_trace_b256_l2048.{md,json}),
      HBM traffic of the fused decode kernel for BF16, INT8 and INT4 pages
      (profiles/decode{,_q8,_q4}_kernel_traffic_b256_l2048.{md,json}, read back
      by bench.py while the kernel sources are unchanged) and, with --util,
      utilisation counters (profiles/decode_kernel_utilisation_b256_l2048.md).

  python bench_profiles.py config N --line FILE --trace DIR --fetch DIR --write DIR --util DIR
      runs of ``bench.py --only-config N``: per candidate launch, the decode
      and merge kernels' average durations, HBM bytes over the algorithmic
      bytes, and utilisation (profiles/decode_step_trace_config*.md; the
      hand-written notes after the notes marker are kept).

  python bench_profiles.py sweep --json FILE --steps K --warmup W
  python bench_profiles.py placement --json FILE --steps K --warmup W
  python bench_profiles.py stream --json FILE --steps K --warmup W
  python bench_profiles.py timeline --json FILE --steps K --warmup W
      the output of ``bench.py --sweep`` / ``--placement-probe`` / ``--page-stream``
      / ``--timeline`` as tables (profiles/decode_step_sweep_workloads_1_6.md,
      profiles/decode_kernel_placement_b256_l2048.md,
      profiles/page_stream_b256_l2048.md,
      profiles/decode_balanced_timeline_workloads_3_4_5.md).

Every mode refuses a run whose kernel sources are not the current ones.

HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what they
read for a 256 MiB device copy of the same run (``--calibration-copy``).
Makes no GPU call.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20
UTIL_COUNTERS = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY "
                 "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES "
                 "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
CLOCK_GHZ = 2.4
CUS = 256
XCDS = 8
HOST = "pa_kernels.h + pa_kernels_q8.h + pa_decode_kernel.h + pa_host.h + "

# the fused decode kernel's instances in the headline run, by format
# (template arguments: page format, BF16 out, append, RoPE, wavefronts per KV
# head, ring slots per wavefront with 0 for the format's default)
HEADLINE_KERNELS = (
    ("void pa::decode_kernel<0, false, true, false, 1, 0>", "BF16",
     "pa::decode_kernel<BF16 pages, FP32 out, append fused>", "TRAFFIC_FILE", "KERNEL_SOURCES",
     "pa_decode.hip", "step_bytes", ""),
    ("void pa::decode_kernel<1, false, true, false, 1, 0>", "INT8",
     "pa::decode_kernel<INT8 pages, FP32 out, quantised append fused>", "TRAFFIC_FILE_Q8",
     "KERNEL_SOURCES_Q8", "pa_decode_q8.hip", "step_bytes_q8", ""),
    ("void pa::decode_kernel<2, false, true, false, 2, 0>", "INT4",
     "pa::decode_kernel<INT4 pages, FP32 out, quantised append fused, two wavefronts per KV head>",
     "TRAFFIC_FILE_Q4", "KERNEL_SOURCES_Q8", "pa_decode_q8.hip", "step_bytes_q4",
     "One 128-page split per sequence, two wavefronts per KV head (each streams 64 pages; the\n"
     "two states merge in LDS), so the kernel writes the outputs directly: no split partials.\n"),
)

TRACE_LABELS = (
    ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<int, at::native::func_wrapper_t"
     "<int, at::native::MaxNanFunctor<int>", "flush (torch amax over 1 GiB)"),
    ("void pa::decode_kernel<0, false, true, false, 1, 0>", "pa::decode_kernel<BF16, append>"),
    ("void pa::decode_kernel<0, false, false, false, 1, 0>", "pa::decode_kernel<BF16, no append>"),
    ("void pa::decode_kernel<0, false, true, true, 1, 0>", "pa::decode_kernel<BF16, append, RoPE>"),
    ("void pa::decode_kernel<0, false, true, false, 1, 2>",
     "pa::decode_kernel<BF16, append, two-slot ring>"),
    ("void pa::decode_kernel<0, false, false, false, 1, 2>",
     "pa::decode_kernel<BF16, no append, two-slot ring>"),
    ("void pa::decode_kernel<1, false, true, false, 1, 0>", "pa::decode_kernel<INT8, append>"),
    ("void pa::decode_kernel<2, false, true, false, 2, 0>",
     "pa::decode_kernel<INT4, append, two wavefronts per KV head>"),
    ("(anonymous namespace)::stream_read_kernel", "pa_stream_read (1 GiB, non-temporal loads)"),
    ("void (anonymous namespace)::page_stream_kernel<0, 1, 1>",
     "pa_page_stream (BF16 pages, decode kernel's shape)"),
    ("void (anonymous namespace)::page_stream_kernel<1, 1, 2>",
     "pa_page_stream (INT8 pages, decode kernel's shape)"),
    ("void (anonymous namespace)::page_stream_kernel<2, 2, 3>",
     "pa_page_stream (INT4 pages, decode kernel's shape)"),
    ("void pa::merge_kernel<false>", "pa::merge_kernel<FP32 out>"),
)


def _csv(d: str, suffix: str):
    hits = sorted(glob.glob(os.path.join(d, f"*_{suffix}.csv")))
    if len(hits) != 1:
        raise SystemExit(f"expected one *_{suffix}.csv under {d}, found {len(hits)}")
    with open(hits[0]) as f:
        return list(csv.DictReader(f))


def _rel(d: str) -> str:
    return os.path.relpath(os.path.abspath(d), ROOT)


def _box(d: str) -> str:
    """A path under the repository as the profiling commands name it: they run
    from /tmp, with the repository at /root/repo."""
    return "/root/repo/" + _rel(d)


def calibration(fetch_rows, write_rows):
    """Counter factors from the 256 MiB device copy: (fetch KiB, write KiB,
    fetch factor, write factor)."""
    w = [r for r in write_rows if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"
         and float(r["Counter_Value"]) > COPY_BYTES / 1024 * 0.75]
    ids = {r["Dispatch_Id"] for r in w}
    f = [r for r in fetch_rows if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"
         and r["Dispatch_Id"] in ids]
    if not w or len(f) != len(w):
        raise SystemExit("no 256 MiB calibration copy in both counter runs "
                         "(run bench.py with --calibration-copy)")
    cw = float(np.mean([float(r["Counter_Value"]) for r in w]))
    cf = float(np.mean([float(r["Counter_Value"]) for r in f]))
    return cf, cw, COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw


def _values(rows, prefix, counter=None):
    return [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith(prefix)
            and (counter is None or r["Counter_Name"] == counter)]


def _label(name: str) -> str:
    for prefix, lab in TRACE_LABELS:
        if name.startswith(prefix):
            return lab
    if "FillFunctor" in name or "arange" in name:
        return "torch fill / arange (input setup)"
    return name.split("(")[0][:70]


def utilisation(rows):
    """Busy shares from one pass of UTIL_COUNTERS over a set of dispatches."""
    per = {}
    for r in rows:
        per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    if not per:
        return None
    n = len(per)
    tot = {c: sum(d.get(c, 0.0) for d in per.values()) for c in UTIL_COUNTERS.split()}
    gui = tot["GRBM_GUI_ACTIVE"] / n / XCDS          # cycles of one XCD per dispatch
    return {
        "dispatches": n,
        "gui_us": gui / (CLOCK_GHZ * 1e3),
        "valu": tot["SQ_ACTIVE_INST_VALU"] / n / CUS / gui,
        "mfma": tot["SQ_VALU_MFMA_BUSY_CYCLES"] / n / CUS / gui,
        "wait": tot["SQ_WAIT_INST_ANY"] / tot["SQ_WAVE_CYCLES"],
        "issue": tot["SQ_ACTIVE_INST_ANY"] / tot["SQ_WAVE_CYCLES"],
        "lds_conflict": (tot["SQ_LDS_BANK_CONFLICT"] / tot["SQ_ACTIVE_INST_LDS"]
                         if tot["SQ_ACTIVE_INST_LDS"] else 0.0),
    }


UTIL_NOTE = ("Counters are summed over the 8 XCDs by rocprofv3; GRBM_GUI_ACTIVE per XCD is the sum / 8.\n"
             "VALU busy and MFMA busy: the counter summed over the device / 256 CUs / GUI-active cycles\n"
             "of one XCD.  Wait and issue shares are of SQ_WAVE_CYCLES (cycles summed over resident\n"
             "waves).  GUI-active µs assumes the 2.4 GHz clock.\n")


def headline(a) -> int:
    import workloads as W  # noqa: F401  (the accounting reads the workload's shapes)
    from paged_kv_decode_07_amd import accounting as A

    lens = np.full(256, 2048)
    line = _json_line(a.line, "kernel_source_sha")
    for key, got in (("BF16", line["kernel_source_sha"]),
                     ("INT8/INT4", line["int8_pages"]["kernel_source_sha"])):
        want = bench.kernel_source_hash(bench.KERNEL_SOURCES if key == "BF16"
                                        else bench.KERNEL_SOURCES_Q8)
        if got != want:
            raise SystemExit(f"the profiled run's {key} kernel sources ({got}) are not the "
                             f"current ones ({want}): profile again")
    cmd_trace = (f"rocprofv3 --kernel-trace --stats -f csv -d {_box(a.trace)} -o bench -- "
                 f"python -u /root/repo/bench.py --steps 20 --warmup 3 --no-cpu-baseline --configs ''")
    cmd_fetch = (f"rocprofv3 --pmc FETCH_SIZE -f csv -d {_box(a.fetch)} -o bench -- python -u "
                 f"/root/repo/bench.py --steps 3 --warmup 1 --no-cpu-baseline --configs '' "
                 f"--calibration-copy")
    cmd_write = cmd_fetch.replace("FETCH_SIZE", "WRITE_SIZE").replace(_box(a.fetch), _box(a.write))
    summary = (f"python bench_profiles.py headline --line {_rel(a.line)} --trace {_rel(a.trace)} "
               f"--fetch {_rel(a.fetch)} "
               f"--write {_rel(a.write)}" + (f" --util {_rel(a.util)}" if a.util else ""))

    fetch, write = _csv(a.fetch, "counter_collection"), _csv(a.write, "counter_collection")
    cf, cw, ff, wf = calibration(fetch, write)
    for prefix, fmt, label, tfile, srcs, hip, acc, note in HEADLINE_KERNELS:
        f, w = _values(fetch, prefix, "FETCH_SIZE"), _values(write, prefix, "WRITE_SIZE")
        if not f or not w:
            raise SystemExit(f"no {fmt} decode dispatches in the counter runs")
        fk, wk = float(np.mean(f)), float(np.mean(w))
        hbm = int(round(fk * 1024 * ff + wk * 1024 * wf))
        sources = getattr(bench, srcs)
        sha = bench.kernel_source_hash(sources)
        alg = getattr(A, acc)(lens, 4, True)
        alg = {k: int(alg[k]) for k in ("kv", "q", "out", "meta", "app", "total")}
        path = getattr(bench, tfile)
        j = {"kernel": label,
             "workload": "batch 256 x 2048 tokens, random page placement, 1 split per sequence",
             "kernel_source_sha": sha, "kernel_sources": HOST + hip,
             "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
             "dispatches": {"fetch": len(f), "write": len(w)},
             "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": round(cf, 4),
                             "copy_write_kib": round(cw, 4), "fetch_factor": round(ff, 5),
                             "write_factor": round(wf, 5)},
             "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
             "algorithmic_total": alg["total"],
             "traffic_over_algorithmic": round(hbm / alg["total"], 5),
             "commands": [cmd_fetch, cmd_write, summary]}
        with open(path, "w") as o:
            json.dump(j, o, indent=1)
            o.write("\n")
        with open(path[:-5] + ".md", "w") as o:
            o.write(f"# HBM traffic counters: {label}, batch 256 x 2048 tokens\n\n")
            o.write("Commands (MI355X, ROCm 7.2; the profiler runs from /tmp with TMPDIR=/tmp, the "
                    "summary from the repository root; two passes, one counter each):\n\n")
            o.write(f"```\n{cmd_fetch}\n{cmd_write}\n{summary}\n```\n\n")
            o.write(f"Kernel sources sha256[:16] = `{sha}` ({HOST}{hip}).\n\n")
            o.write("| quantity | value |\n|---|---|\n")
            o.write(f"| FETCH_SIZE, kernel | {fk:.1f} KiB/dispatch ({len(f)} dispatches) |\n")
            o.write(f"| WRITE_SIZE, kernel | {wk:.1f} KiB/dispatch ({len(w)} dispatches) |\n")
            o.write(f"| FETCH_SIZE, 256 MiB device copy | {cf:.1f} KiB (factor {ff:.4f}) |\n")
            o.write(f"| WRITE_SIZE, 256 MiB device copy | {cw:.1f} KiB (factor {wf:.4f}) |\n")
            o.write(f"| calibrated HBM bytes per launch | {hbm:,} |\n")
            o.write(f"| algorithmic bytes per launch (kv, q, out, meta, app) | {alg['total']:,} |\n")
            o.write(f"| ratio | {hbm / alg['total']:.4f} |\n\n")
            o.write("FETCH_SIZE reads half the bytes of a kernel of known size on this part (the "
                    "256 MiB copy),\nhence the factor 2; WRITE_SIZE is exact.\n")
            if note:
                o.write("\n" + note)
        print(f"{fmt}: {fk:.1f} / {wk:.1f} KiB -> {hbm:,} B vs {alg['total']:,} "
              f"({hbm / alg['total']:.4f})")

    stats = _csv(a.trace, "kernel_stats")
    pass_a = timed_run(_csv(a.trace, "kernel_trace"), HEADLINE_KERNELS[0][0], int(line["steps"]))
    events_us = float(line["roofline"]["avg_launch_us"])
    avg = {}
    kv = {"BF16": int(A.step_bytes(lens)["kv"]), "INT8": int(A.step_bytes_q8(lens)["kv"]),
          "INT4": int(A.step_bytes_q4(lens)["kv"])}
    path = bench.TRACE_FILE[:-5] + ".md"
    with open(path, "w") as o:
        o.write("# Kernel trace: bench.py, batch 256 x 2048 tokens (BF16 pages 1 GiB, INT8 pages "
                "544 MiB, INT4 pages 288 MiB)\n\n")
        o.write("Commands (MI355X, ROCm 7.2; the profiler runs from /tmp with TMPDIR=/tmp, the "
                "summary from the repository root):\n\n")
        o.write(f"```\n{cmd_trace}\n{summary}\n```\n\n")
        o.write(f"Kernel sources sha256[:16] = `{bench.kernel_source_hash(bench.KERNEL_SOURCES)}` "
                f"(BF16: {HOST}pa_decode.hip), "
                f"`{bench.kernel_source_hash(bench.KERNEL_SOURCES_Q8)}` (INT8 and INT4: "
                f"{HOST}pa_decode_q8.hip).\n\n")
        o.write("Passes of the run: fused step (A), two-call step (C), fused step with RoPE (D), "
                "fused step\nover INT8 pages (E), over INT4 pages (F, one split per sequence, two "
                "wavefronts per KV head),\nprefill fill, identity placement, streaming read; every "
                "step follows a 1 GiB read flush.\n\n")
        o.write("| kernel | calls | avg us | min us | max us | share |\n|---|---|---|---|---|---|\n")
        for r in stats:
            lb = _label(r["Name"])
            us = float(r["AverageNs"]) / 1e3
            for prefix, fmt, *_ in HEADLINE_KERNELS:
                if r["Name"].startswith(prefix):
                    avg[fmt] = (us, int(r["Calls"]))
            o.write(f"| {lb} | {r['Calls']} | {us:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                    f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |\n")
        o.write("\n")
        for fmt in ("BF16", "INT8", "INT4"):
            if fmt not in avg:
                raise SystemExit(f"no {fmt} fused decode kernel in the trace")
            us = avg[fmt][0]
            o.write(f"{fmt} fused kernel: {us:.2f} us average -> {kv[fmt] / us / 1e3:.1f} GB/s of "
                    f"{'K/V' if fmt == 'BF16' else 'codes and scales'} "
                    f"({kv[fmt] / us / 1e3 / bench.HBM_PEAK_GBPS * 100:.1f}% of 8 TB/s)"
                    + ("" if fmt == "BF16" else
                       f"; {avg['BF16'][0] / us:.2f}x the BF16 kernel's sequence rate") + ".\n")
        o.write(f"\nThe BF16 fused kernel's {len(pass_a)} timed launches of the headline pass (the "
                f"step is that one launch):\n{pass_a.mean():.2f} us mean (min {pass_a.min():.2f}, "
                f"max {pass_a.max():.2f}) -> {kv['BF16'] / pass_a.mean() / 1e3:.1f} GB/s "
                f"({kv['BF16'] / pass_a.mean() / 1e3 / bench.HBM_PEAK_GBPS * 100:.1f}% of 8 TB/s). "
                f"The same run's events\naround the same launches: {events_us:.2f} us; they also "
                "hold the launch's dispatch after the\nflush kernel, which the trace does not.  "
                "The average over every call above also holds the\nwarm-up and the "
                "identity-placement launches.\n")
    with open(bench.TRACE_FILE, "w") as o:
        json.dump({"kernel": HEADLINE_KERNELS[0][2],
                   "workload": "batch 256 x 2048 tokens, random page placement, 1 split per sequence",
                   "kernel_source_sha": bench.kernel_source_hash(bench.KERNEL_SOURCES),
                   "avg_us": round(float(pass_a.mean()), 3), "calls": len(pass_a),
                   "avg_us_every_call": round(avg["BF16"][0], 3), "every_call": avg["BF16"][1],
                   "bench_events_avg_us": events_us,
                   "algorithmic_kv_bytes": kv["BF16"], "commands": [cmd_trace, summary]}, o, indent=1)
        o.write("\n")
    print(" ".join(f"{k} {v[0]:.2f} us" for k, v in avg.items()))

    if a.util:
        util = _csv(a.util, "counter_collection")
        cmd_util = (f"rocprofv3 --pmc {UTIL_COUNTERS} -f csv -d {_box(a.util)} -o bench -- python -u "
                    f"/root/repo/bench.py --steps 3 --warmup 1 --no-cpu-baseline --configs ''")
        with open(os.path.join(PROFILES, "decode_kernel_utilisation_b256_l2048.md"), "w") as o:
            o.write("# Utilisation counters: pa::decode_kernel, batch 256 x 2048 tokens\n\n")
            o.write("Commands (MI355X, ROCm 7.2; the profiler runs from /tmp with TMPDIR=/tmp, the "
                    "summary from the repository root; one pass):\n\n")
            o.write(f"```\n{cmd_util}\n{summary}\n```\n\n")
            o.write(f"Kernel sources sha256[:16] = `{bench.kernel_source_hash(bench.KERNEL_SOURCES)}` "
                    f"(BF16), `{bench.kernel_source_hash(bench.KERNEL_SOURCES_Q8)}` (INT8 and "
                    "INT4).  The INT4 pass runs one 128-page split per sequence with two wavefronts "
                    "per KV head.\n\n" + UTIL_NOTE + "\n")
            o.write("| kernel | dispatches | GUI-active µs | VALU busy | MFMA busy | waves waiting | "
                    "waves issuing | LDS bank-conflict cycles per LDS-active cycle |\n"
                    "|---|---|---|---|---|---|---|---|\n")
            for prefix, fmt, label, *_ in HEADLINE_KERNELS:
                u = utilisation([r for r in util if r["Kernel_Name"].startswith(prefix)])
                if u is None:
                    raise SystemExit(f"no {fmt} decode dispatches in the utilisation run")
                o.write(f"| {fmt} pages, fused append | {u['dispatches']} | {u['gui_us']:.1f} | "
                        f"{100 * u['valu']:.1f}% | {100 * u['mfma']:.1f}% | {100 * u['wait']:.1f}% | "
                        f"{100 * u['issue']:.1f}% | {u['lds_conflict']:.2f} |\n")
                print(f"{fmt} util: GUI {u['gui_us']:.1f} us VALU {100 * u['valu']:.1f}% "
                      f"MFMA {100 * u['mfma']:.1f}%")
    return 0


def timed_run(trace_rows, prefix: str, steps: int):
    """Durations (us) of the first `steps` consecutive launches of one kernel
    among the library's launches: the timed steps of a pass whose step is that
    one launch (the warm-up steps before them alternate with other launches)."""
    seq = sorted((r for r in trace_rows if "pa::" in r["Kernel_Name"].split("(")[0]),
                 key=lambda r: int(r["Dispatch_Id"]))
    run = []
    for r in seq:
        if r["Kernel_Name"].startswith(prefix):
            run.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            if len(run) == steps:
                return np.array(run)
        else:
            run = []
    raise SystemExit(f"no {steps} consecutive launches of {prefix} in the trace")


def _json_line(path: str, key: str = "launches"):
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and f'"{key}"' in line:
                return json.loads(line)
    raise SystemExit(f"no bench.py JSON line with {key!r} in {path}")


def split_launches(rows, names, layers):
    """The pa:: dispatches of an --only-config run, by candidate launch: every
    candidate runs the same number of steps of `layers` decode launches; a
    merge launch belongs to the candidate whose decode launches precede it."""
    rows = sorted((r for r in rows if "pa::" in r["Kernel_Name"].split("(")[0]),
                  key=lambda r: int(r["Dispatch_Id"]))
    dec_ids = sorted({int(r["Dispatch_Id"]) for r in rows if "decode" in r["Kernel_Name"]})
    per = len(dec_ids) // len(names)
    if per == 0 or per * len(names) != len(dec_ids) or per % layers:
        raise SystemExit(f"{len(dec_ids)} decode dispatches do not split over {len(names)} launches "
                         f"of {layers}-layer steps")
    starts = [dec_ids[k * per] for k in range(len(names))] + [1 << 62]
    out = {n: {"decode": [], "merge": []} for n in names}
    for r in rows:
        i = int(r["Dispatch_Id"])
        k = max(j for j in range(len(names)) if starts[j] <= i) if i >= starts[0] else None
        if k is None:
            continue
        kind = "decode" if "decode" in r["Kernel_Name"] else "merge" if "merge" in r["Kernel_Name"] else None
        if kind:
            out[names[k]][kind].append(r)
    return out


NOTES = "<!-- notes: kept when the tables above are regenerated -->"


def write_keeping_notes(path: str, text: str) -> None:
    """Write a generated summary, keeping whatever an existing file holds after
    the notes marker (the hand-written reading of the tables)."""
    notes = ""
    if os.path.exists(path):
        with open(path) as f:
            old = f.read()
        k = old.find(NOTES)
        if k >= 0:
            notes = old[k + len(NOTES):]
    with open(path, "w") as o:
        o.write(text.rstrip("\n") + "\n\n" + NOTES + (notes if notes else "\n"))


def check_sources(found: dict, keys) -> None:
    want = bench.source_hashes()
    for k in keys:
        if found.get(k) != want[k]:
            raise SystemExit(f"the run's {k} kernel sources ({found.get(k)}) are not the current "
                             f"ones ({want[k]}): run it again")


CONFIG_FILES = {3: "decode_step_trace_config3_b64_16layers.md",
                5: "decode_step_trace_config5_b512_zipf.md"}


def config(a) -> int:
    import workloads as W
    from paged_kv_decode_07_amd import accounting as A

    ci = a.config
    line = _json_line(a.line)
    check_sources(line.get("kernel_sources", {}), ("grid_bf16", "balanced"))
    names = list(line["launches"])
    layers = int(line["layers"])
    alg = A.step_bytes(W.workload_seq_lens(ci), append=True)
    trace = split_launches(_csv(a.trace, "kernel_trace"), names, layers)
    fetch_rows, write_rows = _csv(a.fetch, "counter_collection"), _csv(a.write, "counter_collection")
    cf, cw, ff, wf = calibration(fetch_rows, write_rows)
    fetch = split_launches(fetch_rows, names, layers)
    write = split_launches(write_rows, names, layers)
    util = split_launches(_csv(a.util, "counter_collection"), names, layers) if a.util else None

    def dur(rs):
        return float(np.mean([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                              for r in rs])) if rs else 0.0

    def kib(rs, counter):
        v = [float(r["Counter_Value"]) for r in rs if r["Counter_Name"] == counter]
        return float(np.sum(v)) if v else 0.0

    box = lambda d: _box(d)                                   # noqa: E731
    tag = os.path.basename(os.path.normpath(a.trace))
    cmds = [f"rocprofv3 --kernel-trace --stats -f csv -d {box(a.trace)} -o c{ci} -- python -u "
            f"/root/repo/bench.py --only-config {ci} --steps 10 --warmup 2"]
    for d, ctr in ((a.fetch, "FETCH_SIZE"), (a.write, "WRITE_SIZE")):
        cmds.append(f"rocprofv3 --pmc {ctr} -f csv -d {box(d)} -o c{ci} -- python -u "
                    f"/root/repo/bench.py --only-config {ci} --steps 2 --warmup 1 --calibration-copy")
    if a.util:
        cmds.append(f"rocprofv3 --pmc {UTIL_COUNTERS} -f csv -d {box(a.util)} -o c{ci} -- python -u "
                    f"/root/repo/bench.py --only-config {ci} --steps 2 --warmup 1")
    cmds.append(f"python bench_profiles.py config {ci} --line {_rel(a.line)} --trace {_rel(a.trace)} "
                f"--fetch {_rel(a.fetch)} --write {_rel(a.write)}"
                + (f" --util {_rel(a.util)}" if a.util else ""))
    del tag
    src = line["kernel_sources"]
    out = [f"# Workload {ci}: {W.WORKLOADS[ci]}; fused step, BF16 pages, every launch\n",
           "Commands (MI355X, ROCm 7.2; the profiler runs from /tmp with TMPDIR=/tmp, the summary "
           "from the repository root; one pass each; `--calibration-copy` adds one 256 MiB device "
           "copy as the byte counters' reference):\n",
           "```\n" + "\n".join(cmds) + "\n```\n",
           f"Kernel sources sha256[:16]: grid and work-list kernel `{src['grid_bf16']}`; balanced "
           f"kernel `{src['balanced']}`.\n",
           f"`--only-config {ci}` times the fused append + attention step of the workload's "
           f"{layers} layer{'s' if layers > 1 else ''} back to back under every launch that can "
           "plan it, in this order: " + "; ".join(names) + ". Per layer: K/V "
           f"{int(alg['kv']):,} bytes; every algorithmic byte of the step {int(alg['total']):,}.\n",
           "| launch | work-groups | decode kernel avg us | merge kernel avg us | layer: kernels us "
           "| HBM bytes / algorithmic |\n|---|---|---|---|---|---|"]
    for n in names:
        d, m = trace[n]["decode"], trace[n]["merge"]
        wg = int(d[0]["Grid_Size_X"]) // int(d[0]["Workgroup_Size_X"])
        nd = len(fetch[n]["decode"])
        hbm = ((kib(fetch[n]["decode"] + fetch[n]["merge"], "FETCH_SIZE") * ff
                + kib(write[n]["decode"] + write[n]["merge"], "WRITE_SIZE") * wf) * 1024 / nd)
        dm, mm = dur(d), dur(m)
        per_layer = dm + mm * len(m) / len(d)
        out.append(f"| {n} | {wg} | {dm:.2f} | {mm:.2f} | {per_layer:.2f} | "
                   f"{hbm / float(alg['total']):.4f} |")
    out.append(f"\nHBM bytes: FETCH_SIZE x {ff:.3f} + WRITE_SIZE x {wf:.3f} (KiB per dispatch x "
               f"1024; the 256 MiB copy reads {cf:,.1f} KiB by FETCH_SIZE and writes {cw:,.1f} KiB "
               "by WRITE_SIZE), decode and merge kernels together, per layer.\n")
    if util:
        out.append("Utilisation (decode kernel; " + UTIL_NOTE.replace("\n", " ").strip() + "):\n")
        out.append("| launch | GUI-active us | VALU busy | MFMA busy | waves waiting | waves issuing |\n"
                   "|---|---|---|---|---|---|")
        for n in names:
            u = utilisation(util[n]["decode"])
            out.append(f"| {n} | {u['gui_us']:.1f} | {100 * u['valu']:.1f}% | "
                       f"{100 * u['mfma']:.1f}% | {100 * u['wait']:.1f}% | {100 * u['issue']:.1f}% |")
    text = "\n".join(out) + "\n"
    path = os.path.join(PROFILES, CONFIG_FILES.get(ci, f"decode_step_trace_workload{ci}.md"))
    write_keeping_notes(path, text)
    print(text)
    return 0


def _lines(path: str):
    with open(path) as f:
        return [json.loads(x) for x in f if x.strip().startswith("{")]


def sweep(a) -> int:
    rows = _lines(a.json)
    check_sources(rows[0].get("kernel_sources", {}), ("grid_bf16", "grid_quantised", "balanced"))
    src = rows[0]["kernel_sources"]
    rows = [r for r in rows if "workload" in r]
    out = ["# Fused decode step on every workload: BF16, INT8 and INT4 pages, every launch\n",
           "Commands (MI355X, ROCm 7.2, from the repository root):\n",
           f"```\npython -u bench.py --sweep --steps {a.steps} --warmup {a.warmup} > "
           f"{_rel(a.json)}\npython bench_profiles.py sweep --json {_rel(a.json)} --steps "
           f"{a.steps} --warmup {a.warmup}\n```\n",
           "One layer's fused append + attention step (workload 3: its first layer), caches "
           f"flushed before every step, median of {a.steps} event-timed steps. `grid (lengths "
           "plan)` is `pa_append_decode_attention[_q8|_q4]` with the split size from "
           "`pa_decode_plan_lengths[_q8|_q4]`; `work list` is "
           "`pa_append_decode_attention_worklist[_q8|_q4]` over `pa_decode_worklist`; `balanced, "
           "h KV heads per lane` is `pa_decode_balanced` over `pa_balance_plan` with "
           "`heads_together` = h (work-groups in the units column). K/V bytes: 2,048 per valid "
           "token (BF16 pages), 1,088 (INT8 codes and scales), 576 (INT4). The last rows run "
           "workload 3 as a model step: its 16 layers' fused steps back to back (one pool region "
           "per layer; sequences/s counts the whole 16-layer step), launched as 16 calls and "
           "replayed as one HIP graph. INT4 grid and work-list launches whose grid fits the CUs "
           "with splits of 32 pages or more run two wavefronts per KV head. Kernel sources: grid "
           f"and work list `{src['grid_bf16']}` (BF16) and `{src['grid_quantised']}` (INT8, "
           f"INT4), balanced `{src['balanced']}`.\n",
           "| workload | pages | launch | pages/split | splits, items or work-groups | step µs | "
           "K/V GB/s | sequences/s |\n|---|---|---|---|---|---|---|---|"]
    best = {}
    for r in rows:
        units = r.get("work_groups", r.get("splits", r.get("items", "")))
        rate = r.get("seq_per_s_per_layer", r.get("seq_per_s"))
        out.append(f"| {r['workload']} | {r['pages']} | {r['launch']} | {r['pages_per_split']} | "
                   f"{units} | {r['step_us']} | {r['kv_gbps']:,.0f} | {rate:,.0f} |")
        if "16 calls" in r["launch"] or "graph" in r["launch"]:
            continue
        k = (r["workload"], r["pages"])
        if k not in best or r["step_us"] < best[k]["step_us"]:
            best[k] = r
    out.append("\nFastest launch per workload and page format (one layer):\n")
    out.append("| workload | BF16 | INT8 | INT4 |\n|---|---|---|---|")
    for wi in sorted({k[0] for k in best}):
        cells = []
        for fmt in ("bf16", "int8", "int4"):
            r = best.get((wi, fmt))
            cells.append(f"{r['step_us']} µs, {r['launch']} ({r['kv_gbps']:,.0f} GB/s)" if r else "–")
        out.append(f"| {wi} | " + " | ".join(cells) + " |")
    text = "\n".join(out) + "\n"
    write_keeping_notes(os.path.join(PROFILES, "decode_step_sweep_workloads_1_6.md"), text)
    print(text)
    return 0


def placement(a) -> int:
    rows = _lines(a.json)
    check_sources(rows[0].get("kernel_sources", {}), ("grid_bf16",))
    src = rows[0]["kernel_sources"]
    rows = [r for r in rows if "placement" in r]
    out = ["# Page placement: the decode kernel on batch 256 x 2048 under seven placements\n",
           "Commands (MI355X, ROCm 7.2, from the repository root):\n",
           f"```\npython -u bench.py --placement-probe --steps {a.steps} --warmup {a.warmup} > "
           f"{_rel(a.json)}\npython bench_profiles.py placement --json {_rel(a.json)} --steps "
           f"{a.steps} --warmup {a.warmup}\n```\n",
           "The same logical cache (workload 4 without the append: 256 sequences of 2,048 tokens, "
           "1 GiB of BF16 K/V in a pool of exactly 32,768 pages) is laid out under each placement, "
           "then `pa_decode_attention` (one 128-page split per sequence) runs interleaved over the "
           f"placements, caches flushed before every launch, {a.steps} timed rounds after "
           f"{a.warmup} warm-up rounds; median and minimum of the event-timed launches. "
           "Placements: `identity` (each sequence's pages consecutive, in order); `region` (the "
           "same 128 pages per sequence, shuffled); `chunksN` (random N-page chunks of the pool, "
           "pages shuffled within each chunk); `random` (one random permutation of the pool, the "
           "workload's own placement). Kernel sources "
           f"`{src['grid_bf16']}`.\n",
           "| placement | median µs | min µs | K/V GB/s (median) | output bitwise = identity |\n"
           "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['placement']} | {r['decode_us_median']:.2f} | {r['decode_us_min']:.2f} | "
                   f"{r['kv_gbps']:,.1f} | {r['same_output_as_identity']} |")
    med = [r["decode_us_median"] for r in rows]
    out.append(f"\nThe spread is {100 * (max(med) / min(med) - 1):.1f}% "
               f"({min(med):.1f} to {max(med):.1f} µs).")
    text = "\n".join(out) + "\n"
    write_keeping_notes(os.path.join(PROFILES, "decode_kernel_placement_b256_l2048.md"), text)
    print(text)
    return 0


def stream(a) -> int:
    rows = _lines(a.json)
    check_sources(rows[0].get("kernel_sources", {}), ("grid_bf16", "grid_quantised", "page_stream"))
    src = rows[0]["kernel_sources"]
    rows = [r for r in rows if "case" in r]
    out = ["# Page stream: each format's page reads alone, beside its decode kernel, batch 256 x 2048\n",
           "Commands (MI355X, ROCm 7.2, from the repository root):\n",
           f"```\npython -u bench.py --page-stream --steps {a.steps} --warmup {a.warmup} > "
           f"{_rel(a.json)}\npython bench_profiles.py stream --json {_rel(a.json)} --steps "
           f"{a.steps} --warmup {a.warmup}\n```\n",
           "Workload 4 without the append (256 sequences of 2,048 tokens at random pool slots). "
           "`decode kernel` is `pa_decode_attention[_q8|_q4]` with the library's default plan "
           "(one 128-page split per sequence). `page stream` is `pa_page_stream`: the same pages "
           "requested with the decode kernel's direct-to-LDS loads for that format (same "
           "lane-to-address maps, non-temporal policy and ring waits), each landed page read back "
           "from LDS and folded, nothing else computed, with h wavefronts per KV head and an LDS "
           "ring of r slots per wavefront; `*` marks the decode kernel's own (h, r). All cases "
           f"run interleaved, caches flushed before every launch, {a.steps} timed rounds after "
           f"{a.warmup} warm-up rounds; median and minimum of the event-timed launches. Bytes: "
           "the K/V (and scale) bytes of the batch, 1 GiB BF16, 544 MiB INT8, 288 MiB INT4. "
           f"Kernel sources: decode `{src['grid_bf16']}` (BF16), `{src['grid_quantised']}` (INT8, "
           f"INT4); page stream `{src['page_stream']}`.\n",
           "| format | case | h | r | median µs | min µs | GB/s (median) | % of 8 TB/s |\n"
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        own = "*" if r.get("decode_kernel_shape") else ""
        h = r.get("waves_per_head", "")
        rr = f"{r['ring']}{own}" if "ring" in r else ""
        out.append(f"| {r['format']} | {r['case']} | {h} | {rr} | {r['us_median']:.2f} | "
                   f"{r['us_min']:.2f} | {r['gbps']:,.1f} | {100 * r['frac_of_peak']:.1f} |")
    out.append("\nEach decode kernel beside the stream of its own shape and the fastest stream:\n")
    out.append("| format | decode µs | own stream µs | decode / own stream | fastest stream (h, r) µs "
               "| decode / fastest |\n|---|---|---|---|---|---|")
    for fmt in ("bf16", "int8", "int4"):
        dec = [r for r in rows if r["format"] == fmt and r["case"] == "decode kernel"]
        st = [r for r in rows if r["format"] == fmt and r["case"] == "page stream"]
        own = [r for r in st if r.get("decode_kernel_shape")]
        if not dec or not own:
            continue
        fast = min(st, key=lambda r: r["us_median"])
        d, o = dec[0]["us_median"], own[0]["us_median"]
        out.append(f"| {fmt} | {d:.2f} | {o:.2f} | {d / o:.3f} | ({fast['waves_per_head']}, "
                   f"{fast['ring']}) {fast['us_median']:.2f} | {d / fast['us_median']:.3f} |")
    text = "\n".join(out) + "\n"
    write_keeping_notes(os.path.join(PROFILES, "page_stream_b256_l2048.md"), text)
    print(text)
    return 0


def timeline(a) -> int:
    rows = _lines(a.json)
    check_sources(rows[0].get("kernel_sources", {}), ("balanced",))
    src = rows[0]["kernel_sources"]
    rows = [r for r in rows if "case" in r]
    khz = rows[0]["clock_khz"]
    out = ["# Timeline of the balanced launch: where a launch's time goes, workloads 3, 4 and 5\n",
           "Commands (MI355X, ROCm 7.2, from the repository root):\n",
           f"```\npython -u bench.py --timeline --steps {a.steps} --warmup {a.warmup} > "
           f"{_rel(a.json)}\npython bench_profiles.py timeline --json {_rel(a.json)} --steps "
           f"{a.steps} --warmup {a.warmup}\n```\n",
           "`pa_decode_balanced_timeline` runs the balanced launch's own kernel body (the same "
           "reads, arithmetic and writes, outputs equal bit for bit) and stamps every wavefront "
           f"with the device's real-time counter ({khz / 1000:g} MHz by `pa_wall_clock_khz`) at "
           "its start, when its plan descriptor is in, when the lengths, page ids and q rows are "
           "in, when its first page is in LDS, when its last page is consumed, and when its output "
           "stores are issued and acknowledged. Fused append + attention, FP32 out, each step's "
           "layers back to back on one stream, caches flushed before every step; timeline and "
           f"plain steps interleaved, {a.steps} of each after {a.warmup} warm-up rounds. Phases "
           "are medians over every wavefront of every launch of the timed steps; `pages` are the "
           "pages of one wavefront's KV-head stream (4 KiB of BF16 K and V each). Workload 4 runs "
           "here with 8 heads per lane (one sequence per work-group), the same shape as its grid "
           f"launch. Balanced kernel sources `{src['balanced']}`.\n",
           "| case | work-groups | plain step µs (per layer) | timeline step µs | launch span µs "
           "| gap to next layer µs | start spread µs | descriptor µs | lengths, ids, q µs "
           "| then first page µs | first page at µs | stream µs | µs per page | tail µs |\n"
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    f = lambda v, d=2: "–" if v is None else f"{v:.{d}f}"
    for r in rows:
        out.append(f"| {r['case']} | {r['groups']} | {r['step_us_plain']:.1f} "
                   f"({r['per_layer_us_plain']:.2f}) | {r['step_us_timeline']:.1f} | "
                   f"{f(r['span_us'])} | {f(r['gap_us'])} | {f(r['dispatch_us'])} | "
                   f"{f(r['descriptor_us'])} | {f(r['metadata_us'])} | {f(r['first_page_us'])} | "
                   f"{f(r['first_page_at_us'])} | {f(r['stream_us'])} | {f(r['us_per_page'], 3)} | "
                   f"{f(r['tail_us'])} |")
    out.append("\nWork-group end times (µs after the launch's first wavefront started, every "
               "work-group of every launch) and the pages per wavefront:\n")
    out.append("| case | min | p10 | median | p90 | max | max - median | pages per wavefront "
               "(min / median / max) | stamped / event time |\n|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        e = r["wg_end_us"]
        pw = r["pages_per_wave"]
        out.append(f"| {r['case']} | {e['min']:.2f} | {e['p10']:.2f} | {e['p50']:.2f} | "
                   f"{e['p90']:.2f} | {e['max']:.2f} | {e['max'] - e['p50']:.2f} | {pw['min']} / "
                   f"{pw['median']:g} / {pw['max']} | {r['stamped_over_event']:.3f} |")
    out.append("\nBy die (the XCC_ID each work-group ran on): median work-group end µs / median "
               "µs per page:\n")
    ids = sorted({k for r in rows for k in r["by_xcc"]}, key=int)
    out.append("| case | " + " | ".join(f"XCD {k}" for k in ids) + " |\n|---|" +
               "---|" * len(ids))
    for r in rows:
        cells = [f"{r['by_xcc'][k]['wg_end_median_us']:.2f} / {r['by_xcc'][k]['us_per_page']:.3f}"
                 if k in r["by_xcc"] else "–" for k in ids]
        out.append(f"| {r['case']} | " + " | ".join(cells) + " |")
    text = "\n".join(out) + "\n"
    write_keeping_notes(os.path.join(PROFILES, "decode_balanced_timeline_workloads_3_4_5.md"),
                        text)
    print(text)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    h = sub.add_parser("headline")
    h.add_argument("--line", required=True,
                   help="a file holding the JSON line of the traced bench.py run (its kernel "
                        "source hashes must be the current ones)")
    c = sub.add_parser("config")
    c.add_argument("config", type=int)
    c.add_argument("--line", required=True,
                   help="a file holding the JSON line of the traced bench.py --only-config run")
    for p in (h, c):
        p.add_argument("--trace", required=True)
        p.add_argument("--fetch", required=True)
        p.add_argument("--write", required=True)
        p.add_argument("--util", default=None)
    for name, flag in (("sweep", "sweep"), ("placement", "placement-probe"),
                       ("stream", "page-stream"), ("timeline", "timeline")):
        p = sub.add_parser(name)
        p.add_argument("--json", required=True, help=f"the output of bench.py --{flag}")
        p.add_argument("--steps", type=int, required=True)
        p.add_argument("--warmup", type=int, required=True)
    a = ap.parse_args(argv)
    return {"headline": headline, "config": config, "sweep": sweep, "placement": placement,
            "stream": stream, "timeline": timeline}[a.mode](a)


if __name__ == "__main__":
    sys.exit(main())
