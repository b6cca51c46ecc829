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

