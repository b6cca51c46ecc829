"""Summaries under profiles/ from rocprofv3 runs of bench.py.

Two modes, each reading rocprofv3 output directories (``-f csv -d DIR``):

  python bench_profiles.py headline --line FILE --trace DIR --fetch DIR --write DIR [--util DIR]
      runs of ``bench.py --no-cpu-baseline --configs ''`` (the batch 256 x 2048
      line): the kernel trace (profiles/decode_kernel_trace_b256_l2048.{md,json}),
      HBM traffic of the fused decode kernel for BF16, INT8 and INT4 pages
      (profiles/decode{,_q8,_q4}_kernel_traffic_b256_l2048.{md,json}, read back
      by bench.py while the kernel sources are unchanged) and, with --util,
      utilisation counters (profiles/decode_kernel_utilisation_b256_l2048.md).

  python bench_profiles.py config N --trace DIR --fetch DIR --write DIR --util DIR
      runs of ``bench.py --only-config N``: per candidate launch, the decode
      and merge kernels' average durations, HBM bytes over the algorithmic
      bytes, and utilisation; prints a markdown table (the profile's prose is
      written around it).

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
# (template arguments: page format, BF16 out, append, RoPE, wavefronts per KV head)
HEADLINE_KERNELS = (
    ("void pa::decode_kernel<0, false, true, false, 1>", "BF16",
     "pa::decode_kernel<BF16 pages, FP32 out, append fused>", "TRAFFIC_FILE", "KERNEL_SOURCES",
     "pa_decode.hip", "step_bytes", ""),
    ("void pa::decode_kernel<1, false, true, false, 1>", "INT8",
     "pa::decode_kernel<INT8 pages, FP32 out, quantised append fused>", "TRAFFIC_FILE_Q8",
     "KERNEL_SOURCES_Q8", "pa_decode_q8.hip", "step_bytes_q8", ""),
    ("void pa::decode_kernel<2, false, true, false, 2>", "INT4",
     "pa::decode_kernel<INT4 pages, FP32 out, quantised append fused, two wavefronts per KV head>",
     "TRAFFIC_FILE_Q4", "KERNEL_SOURCES_Q8", "pa_decode_q8.hip", "step_bytes_q4",
     "One 128-page split per sequence, two wavefronts per KV head (each streams 64 pages; the\n"
     "two states merge in LDS), so the kernel writes the outputs directly: no split partials.\n"),
)

TRACE_LABELS = (
    ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<int, at::native::func_wrapper_t"
     "<int, at::native::MaxNanFunctor<int>", "flush (torch amax over 1 GiB)"),
    ("void pa::decode_kernel<0, false, true, false, 1>", "pa::decode_kernel<BF16, append>"),
    ("void pa::decode_kernel<0, false, false, false, 1>", "pa::decode_kernel<BF16, no append>"),
    ("void pa::decode_kernel<0, false, true, true, 1>", "pa::decode_kernel<BF16, append, RoPE>"),
    ("void pa::decode_kernel<1, false, true, false, 1>", "pa::decode_kernel<INT8, append>"),
    ("void pa::decode_kernel<2, false, true, false, 2>",
     "pa::decode_kernel<INT4, append, two wavefronts per KV head>"),
    ("(anonymous namespace)::stream_read_kernel", "pa_stream_read (1 GiB, non-temporal loads)"),
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


def config(a) -> int:
    import workloads as W
    from paged_kv_decode_07_amd import accounting as A

    ci = a.config
    line = _json_line(a.line)
    names = list(line["launches"])
    layers = int(line["layers"])
    alg = A.step_bytes(W.workload_seq_lens(ci), append=True)
    trace = split_launches(_csv(a.trace, "kernel_trace"), names, layers)
    fetch_rows, write_rows = _csv(a.fetch, "counter_collection"), _csv(a.write, "counter_collection")
    _, _, ff, wf = calibration(fetch_rows, write_rows)
    fetch = split_launches(fetch_rows, names, layers)
    write = split_launches(write_rows, names, layers)
    util = split_launches(_csv(a.util, "counter_collection"), names, layers) if a.util else None

    def dur(rs):
        return float(np.mean([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                              for r in rs])) if rs else 0.0

    def kib(rs, counter):
        v = [float(r["Counter_Value"]) for r in rs if r["Counter_Name"] == counter]
        return float(np.sum(v)) if v else 0.0

    print(f"config {ci}: {layers} layer(s); per layer K/V {int(alg['kv']):,} B, every algorithmic "
          f"byte {int(alg['total']):,} B\n")
    print("| launch | work-groups | decode kernel avg us | merge kernel avg us | layer: kernels us "
          "| HBM bytes / algorithmic |\n|---|---|---|---|---|---|")
    for n in names:
        d, m = trace[n]["decode"], trace[n]["merge"]
        wg = int(d[0]["Grid_Size_X"]) // int(d[0]["Workgroup_Size_X"])
        nd = len(fetch[n]["decode"])
        hbm = ((kib(fetch[n]["decode"] + fetch[n]["merge"], "FETCH_SIZE") * ff
                + kib(write[n]["decode"] + write[n]["merge"], "WRITE_SIZE") * wf) * 1024 / nd)
        dm, mm = dur(d), dur(m)
        per_layer = dm + mm * len(m) / len(d)
        print(f"| {n} | {wg} | {dm:.2f} | {mm:.2f} | {per_layer:.2f} | "
              f"{hbm / float(alg['total']):.4f} |")
    if util:
        print("\n| launch | GUI-active us | VALU busy | MFMA busy | waves waiting | waves issuing |\n"
              "|---|---|---|---|---|---|")
        for n in names:
            u = utilisation(util[n]["decode"])
            print(f"| {n} | {u['gui_us']:.1f} | {100 * u['valu']:.1f}% | {100 * u['mfma']:.1f}% | "
                  f"{100 * u['wait']:.1f}% | {100 * u['issue']:.1f}% |")
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
    a = ap.parse_args(argv)
    return headline(a) if a.mode == "headline" else config(a)


if __name__ == "__main__":
    sys.exit(main())
