"""bench.py's host-side logic, without a GPU: the calibrated HBM-traffic summary from
rocprofv3 counter files, the source-hash guard on a stored traffic figure, and the
one-GPU contract."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_pmc_scales_each_counter_by_the_copy(tmp_path):
    interp = "void mk::interpreter_kernel<mk::Spec<true, true, 1, 8, 28> >(mk::LaunchArgs)"
    copy = "copy16_kernel(HIP_vector_type<unsigned int, 4u> const*, HIP_vector_type<unsigned int, 4u>*, unsigned long)"
    # A 1 MiB copy whose fetch counter reads half its bytes (scale 2) and whose write
    # counter reads all of them (scale 1); the interpreter's medians are 1000 and 10 KiB.
    _counter_csv(str(tmp_path / "f"), "FETCH_SIZE",
                 [(interp, 999), (interp, 1000), (interp, 1001), (copy, 512), (copy, 512), ("other", 7)])
    _counter_csv(str(tmp_path / "w"), "WRITE_SIZE", [(interp, 10), (interp, 10), (copy, 1024)])
    t = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), 1 << 20, "8b_b1", "cmd")
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["traffic_bytes_per_launch"] == 1000 * 1024 * 2 + 10 * 1024
    assert t["launches"] == [3, 2] and t["kernel_source_hash"] == bench.kernel_source_hash()


def test_stored_traffic_needs_the_same_kernel_sources(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(path))
    path.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "traffic_bytes_per_launch": 5.0}))
    assert bench.measured_traffic("8b_b1") == 5.0
    path.write_text(json.dumps({"kernel_source_hash": "0" * 16, "traffic_bytes_per_launch": 5.0}))
    assert bench.measured_traffic("8b_b1") is None


def test_committed_traffic_summary_is_plausible():
    # Counter bytes at least the algorithmic bytes of the step (15.278 GB) and not far
    # above them; whether it still matches the kernel sources is bench.py's check.
    with open(bench.traffic_path("8b_b1")) as f:
        t = json.load(f)
    assert 1.0 <= t["traffic_bytes_per_launch"] / 15_278_292_992 < 1.2
    assert t["launches"][0] > 0 and t["launches"][1] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stdout
