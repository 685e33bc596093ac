"""Host logic of bench.py (no GPU): the traffic figure and its staleness rule, the counter
summary arithmetic, and the one-GPU guard."""

import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _counter_csv(path, counter, rows):
    """A rocprofv3 counter CSV with the columns write_traffic reads: rows of
    (dispatch id, kernel name, grid size, value); a dispatch may span several rows."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for d, name, grid, value in rows:
            w.writerow([d, name, grid, counter, value])


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    attn = "void sa::sparse_attn_mfma<128, true>(unsigned short const*, ...)"
    copy = "__amd_rocclr_copyBuffer"
    # the 1 GiB copy reads 524,288 KiB of FETCH_SIZE (factor 2) and 1,048,576 of WRITE_SIZE;
    # two whole-T attention launches (one split over two rows) and one half-range launch
    _counter_csv(str(tmp_path / "fetch" / "f_counter_collection.csv"), "FETCH_SIZE", [
        (1, copy, 4096, 524288.0), (2, attn, 4194304, 600.0), (2, attn, 4194304, 400.0),
        (3, attn, 4194304, 3000.0), (4, attn, 2097152, 99999.0)])
    _counter_csv(str(tmp_path / "write" / "w_counter_collection.csv"), "WRITE_SIZE", [
        (1, copy, 4096, 1048576.0), (2, attn, 4194304, 10.0), (3, attn, 4194304, 30.0),
        (4, attn, 2097152, 77777.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    t = bench.write_traffic(str(tmp_path))
    assert t["fetch_factor"] == 2.0 and t["write_factor"] == 1.0
    assert t["fetch_kib_per_launch"] == 2000.0 and t["write_kib_per_launch"] == 20.0
    assert t["bytes_per_launch"] == 2000.0 * 1024 * 2 + 20.0 * 1024
    assert json.loads(out.read_text())["source_sha256"] == bench.attn_sources_hash()


def test_measured_traffic_is_null_once_the_sources_change(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"source_sha256": bench.attn_sources_hash(),
                               "bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic() == 123.0
    monkeypatch.setattr(bench, "attn_sources_hash", lambda: "0" * 64)
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert json.loads(r.stdout.strip().splitlines()[-1])["n_gpus"] == 2
