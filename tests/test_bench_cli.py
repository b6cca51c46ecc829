"""bench.py's command-line contract that holds without a GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"kernel_source_sha": "0" * 16, "hbm_bytes_per_launch": 1.0}))
    assert bench.measured_traffic(str(f)) is None
    f.write_text(json.dumps({"kernel_source_sha": bench.kernel_source_hash(),
                             "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic(str(f)) == 123
    # the INT8 kernel's figure is keyed to the INT8 sources
    assert bench.measured_traffic(str(f), bench.KERNEL_SOURCES_Q8) is None
    f.write_text(json.dumps({"kernel_source_sha": bench.kernel_source_hash(bench.KERNEL_SOURCES_Q8),
                             "hbm_bytes_per_launch": 7.0}))
    assert bench.measured_traffic(str(f), bench.KERNEL_SOURCES_Q8) == 7


def test_config_lists_are_checked_before_any_work():
    for bad in (["--configs", "4"], ["--configs", "1,7"], ["--configs", "x"],
                ["--only-config", "6"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *bad],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (bad, r.stderr)
    sys.path.insert(0, ROOT)
    import bench
    assert bench.parse_configs("5,1,3,3") == [1, 3, 5]
    assert bench.parse_configs("") == []


def test_rocprof_time_is_dropped_when_the_kernel_changed(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"kernel_source_sha": "0" * 16, "avg_us": 160.0,
                             "algorithmic_kv_bytes": 1 << 30}))
    assert bench.rocprof_kernel_time(str(f)) is None
    f.write_text(json.dumps({"kernel_source_sha": bench.kernel_source_hash(), "avg_us": 160.0,
                             "algorithmic_kv_bytes": 1 << 30, "calls": 20}))
    r = bench.rocprof_kernel_time(str(f))
    assert r["avg_us"] == 160.0 and abs(r["achieved"] - (1 << 30) / 160e3) < 0.01
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4


def test_oracle_rates_and_parity_on_the_host():
    sys.path.insert(0, ROOT)
    import bench
    bench.prepare_states([1], "random")
    r = bench.oracle_rates(1, 0.2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["seq_per_s"] > 0
    refs = bench.oracle_refs(1)
    bumped = [x.copy() for x in refs]
    bumped[0][0, 3, 5] += 1e-3
    err, rel = bench.parity(bumped, refs)
    assert abs(err - 1e-3) < 1e-12 and rel > 0


def test_placement_probe_tables_hold_every_page_once():
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    for scheme in ("identity", "region", "chunks4", "chunks16", "chunks32", "chunks64", "random"):
        t = bench.placement_tables(16, 128, scheme)
        assert t.shape == (16, 128)
        assert np.array_equal(np.sort(t.reshape(-1)), np.arange(16 * 128)), scheme
    assert np.array_equal(bench.placement_tables(4, 128, "identity")[2], np.arange(256, 384))
    reg = bench.placement_tables(4, 128, "region")
    assert all(set(reg[b]) == set(range(128 * b, 128 * b + 128)) for b in range(4))
    ch = bench.placement_tables(4, 128, "chunks16").reshape(-1, 16)
    assert all(len(set(c // 16)) == 1 for c in ch)     # each 16 logical pages: one chunk


def test_profile_summaries_split_launches_and_calibrate(tmp_path):
    sys.path.insert(0, ROOT)
    import bench_profiles as P

    def row(i, name, counter="FETCH_SIZE", value=1.0):
        return {"Dispatch_Id": str(i), "Kernel_Name": name, "Counter_Name": counter,
                "Counter_Value": str(value)}
    dec, mer = "void pa::decode_kernel<0, false, true, false, 1, 0>(pa::DecodeArgs)", \
        "void pa::merge_kernel<false>(pa::MergeArgs)"
    bal = "void pa::decode_balanced_kernel<0, false, true, false, 0>(pa::BalancedArgs)"
    # two launches, 2 steps of 2 layers each; the first has a merge after every decode
    rows = [row(1, "torch fill")]
    i = 2
    for _ in range(4):
        rows += [row(i, dec), row(i + 1, mer)]
        i += 2
    rows += [row(i + k, bal) for k in range(4)]
    s = P.split_launches(rows, ["grid", "balanced"], 2)
    assert [len(s["grid"]["decode"]), len(s["grid"]["merge"])] == [4, 4]
    assert [len(s["balanced"]["decode"]), len(s["balanced"]["merge"])] == [4, 0]
    try:
        P.split_launches(rows, ["a", "b", "c"], 1)
    except SystemExit:
        pass
    else:
        raise AssertionError("8 decode launches over 3 candidates must be refused")
    # calibration: the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all
    copy = "__amd_rocclr_copyBuffer"
    f = [row(7, copy, "FETCH_SIZE", 131072.0), row(8, copy, "FETCH_SIZE", 2.0)]
    w = [row(7, copy, "WRITE_SIZE", 262144.0), row(8, copy, "WRITE_SIZE", 4.0)]
    cf, cw, ff, wf = P.calibration(f, w)
    assert (cf, cw) == (131072.0, 262144.0) and abs(ff - 2.0) < 1e-12 and abs(wf - 1.0) < 1e-12


def test_profile_summary_refuses_a_run_of_other_sources(tmp_path):
    sys.path.insert(0, ROOT)
    import bench_profiles as P
    line = tmp_path / "run.log"
    line.write_text("[bench] noise\n" + json.dumps({"kernel_source_sha": "0" * 16,
                                                   "int8_pages": {"kernel_source_sha": "1" * 16}})
                    + "\n")
    for d in ("t", "f", "w"):
        (tmp_path / d).mkdir()
    try:
        P.main(["headline", "--line", str(line), "--trace", str(tmp_path / "t"),
                "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w")])
    except SystemExit as e:
        assert "profile again" in str(e)
    else:
        raise AssertionError("a run of other kernel sources must be refused")


def test_profile_summaries_keep_the_notes_and_refuse_other_sources(tmp_path):
    sys.path.insert(0, ROOT)
    import bench_profiles as P
    f = tmp_path / "p.md"
    P.write_keeping_notes(str(f), "# tables v1\n")
    assert f.read_text().startswith("# tables v1") and P.NOTES in f.read_text()
    f.write_text(f.read_text() + "- a reading of the tables\n")
    P.write_keeping_notes(str(f), "# tables v2\n")
    text = f.read_text()
    assert text.startswith("# tables v2") and "v1" not in text
    assert text.endswith(P.NOTES + "\n- a reading of the tables\n")
    j = tmp_path / "sweep.json"
    j.write_text(json.dumps({"kernel_sources": {"grid_bf16": "0", "grid_quantised": "1",
                                                "balanced": "2"}}) + "\n")
    try:
        P.main(["sweep", "--json", str(j), "--steps", "1", "--warmup", "1"])
    except SystemExit as e:
        assert "run it again" in str(e)
    else:
        raise AssertionError("a sweep of other kernel sources must be refused")


def test_kernel_hash_ignores_comments_but_not_code(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    a = tmp_path / "a.h"
    a.write_text("// a kernel\nint f(int x) {\n  return x + 1;  /* one */\n}\n")
    h0 = bench.kernel_source_hash([str(a)])
    a.write_text("// the kernel, reworded\n\nint f(int x) {\n  return x + 1;  /* the one */\n}\n")
    assert bench.kernel_source_hash([str(a)]) == h0
    a.write_text("// a kernel\nint f(int x) {\n  return x + 2;  /* one */\n}\n")
    assert bench.kernel_source_hash([str(a)]) != h0


def test_page_stream_summary_sets_each_kernel_beside_its_own_stream(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    import bench_profiles as P
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    rows = [{"kernel_sources": bench.source_hashes()}]
    for fmt, dec, own, fast in (("bf16", 160.0, 158.0, 157.0), ("int8", 88.0, 86.0, 85.0),
                                ("int4", 52.0, 50.0, 47.0)):
        rows.append({"format": fmt, "case": "decode kernel", "us_median": dec, "us_min": dec - 1,
                     "gbps": 1.0, "frac_of_peak": 0.5, "steps": 3})
        wph, ring = bench.STREAM_SHAPES[fmt]
        for (h, r), t in (((wph, ring), own), ((2, 2), fast)):
            rows.append({"format": fmt, "case": "page stream", "us_median": t, "us_min": t - 1,
                         "gbps": 1.0, "frac_of_peak": 0.5, "steps": 3, "waves_per_head": h,
                         "ring": r, "decode_kernel_shape": (h, r) == (wph, ring)})
    j = tmp_path / "stream.json"
    j.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    assert P.main(["stream", "--json", str(j), "--steps", "3", "--warmup", "1"]) == 0
    text = (tmp_path / "page_stream_b256_l2048.md").read_text()
    assert "| int4 | 52.00 | 50.00 | 1.040 | (2, 2) 47.00 | 1.106 |" in text
    assert "| bf16 | 160.00 | 158.00 | 1.013 | (2, 2) 157.00 | 1.019 |" in text
    rows[0] = {"kernel_sources": {**bench.source_hashes(), "page_stream": "0" * 16}}
    j.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    try:
        P.main(["stream", "--json", str(j), "--steps", "3", "--warmup", "1"])
    except SystemExit as e:
        assert "run it again" in str(e)
    else:
        raise AssertionError("a page-stream run of other sources must be refused")


def _hand_stamps():
    """Two work-groups of 8 wavefronts, 100 ticks per µs: start 10 + g + w ticks,
    then 0.3, 1.8, 1.4 µs, 1 µs per page over 11 pages, 0.5 and 1.2 µs; wavefront
    (1, 7) has no pages."""
    import numpy as np
    st = np.zeros((2, 8, 8), np.int64)
    for g in range(2):
        for w in range(8):
            pages = 0 if (g, w) == (1, 7) else 11
            t0 = 10 + g + w
            t1, t2 = t0 + 30, t0 + 210
            t3 = t2 + 140 if pages else 0
            t4 = t3 + 100 * (pages - 1) if pages else t2
            t5 = t4 + 50
            st[g, w, :7] = (t0, t1, t2, t3, t4, t5, t5 + 120)
            st[g, w, 7] = (pages << 48) | (g << 32) | 0x1234
    return st


def test_timeline_phases_from_hand_made_stamps():
    sys.path.insert(0, ROOT)
    import bench
    p = bench.timeline_phases(_hand_stamps(), 100_000.0)
    assert abs(p["descriptor_us"] - 0.3) < 1e-9 and abs(p["metadata_us"] - 1.8) < 1e-9
    assert abs(p["first_page_us"] - 1.4) < 1e-9 and abs(p["us_per_page"] - 1.0) < 1e-9
    assert abs(p["stream_us"] - 10.0) < 1e-9 and abs(p["tail_us"] - 1.7) < 1e-9
    assert abs(p["dispatch_us"] - 0.08) < 1e-9                 # starts 10 .. 18 ticks
    assert abs(p["span_us"] - (17 + 210 + 140 + 1000 + 170 - 10) / 100) < 1e-9
    assert abs(p["first_page_at_us"] - (p["descriptor_us"] + p["metadata_us"] + 1.4 + 0.035)) < 0.05
    assert list(p["xcc"]) == [0, 1]
    assert abs(p["wg_end_us"] - 15.27).max() < 1e-9            # both end with a 11-page wave at 17


def test_timeline_summary_tables(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    import bench_profiles as P
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    rows = [{"kernel_sources": bench.source_hashes()}]
    for ci, h, nl in ((3, 1, 16), (4, 8, 1)):
        rows.append({"case": f"workload {ci}, balanced, {h} KV heads per lane", "workload": ci,
                     "layers": nl, "batch": 64, "heads_together": h, "groups": 256, "steps": 3,
                     "warmup": 1, "clock_khz": 100000, "step_us_timeline": 441.0,
                     "step_us_plain": 437.0, "per_layer_us_plain": 437.0 / nl,
                     "gap_us": 1.4 if nl > 1 else None, "span_us": 25.7, "dispatch_us": 0.3,
                     "descriptor_us": 0.28, "metadata_us": 1.76, "first_page_us": 1.44,
                     "first_page_at_us": 3.66, "stream_us": 16.0, "us_per_page": 1.131,
                     "tail_us": 1.72,
                     "wg_end_us": {"min": 19.5, "p10": 21.1, "p50": 22.2, "p90": 24.4, "max": 25.7},
                     "by_xcc": {"0": {"wg_end_median_us": 21.3, "us_per_page": 1.043,
                                      "work_groups": 32},
                                "3": {"wg_end_median_us": 24.8, "us_per_page": 1.337,
                                      "work_groups": 32}},
                     "pages_per_wave": {"min": 9, "median": 15.0, "max": 16},
                     "stamped_over_event": 0.99})
    j = tmp_path / "timeline.json"
    j.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    assert P.main(["timeline", "--json", str(j), "--steps", "3", "--warmup", "1"]) == 0
    text = (tmp_path / "decode_balanced_timeline_workloads_3_4_5.md").read_text()
    assert ("| workload 3, balanced, 1 KV heads per lane | 256 | 437.0 (27.31) | 441.0 | 25.70 | "
            "1.40 | 0.30 | 0.28 | 1.76 | 1.44 | 3.66 | 16.00 | 1.131 | 1.72 |") in text
    assert "| workload 4, balanced, 8 KV heads per lane | 256 | 437.0 (437.00) | 441.0 | 25.70 | – |" in text
    assert "| 19.50 | 21.10 | 22.20 | 24.40 | 25.70 | 3.50 | 9 / 15 / 16 | 0.990 |" in text
    assert "| XCD 0 | XCD 3 |" in text and "| 21.30 / 1.043 | 24.80 / 1.337 |" in text
    rows[0] = {"kernel_sources": {**bench.source_hashes(), "balanced": "0" * 16}}
    j.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    try:
        P.main(["timeline", "--json", str(j), "--steps", "3", "--warmup", "1"])
    except SystemExit as e:
        assert "run it again" in str(e)
    else:
        raise AssertionError("a timeline run of other sources must be refused")
