"""Host-side logic of bench.py, on the CPU: the counter-traffic summary (each
counter scaled by what it reads for a copy of known size), the guard that drops
counter figures taken on other kernel sources, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def _row(name, grid, value):
    return {"Kernel_Name": name, "Grid_Size": grid, "Counter_Value": value}


def test_summarize_pmc_scales_each_counter_by_the_copy(tmp_path):
    dom = "void " + bench.DOMINANT + "(saga::SelectArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # a 4 MiB copy: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them; small
    # copies (below a quarter of the known size) and other kernels are ignored
    fetch = [_row(copy, 1, 2048.0)] * 3 + [_row(copy, 1, 16.0)] + \
        [_row(dom, 1024, v) for v in (99.0, 100.0, 101.0)] + [_row("other", 8, 1e9)]
    write = [_row(copy, 1, 4096.0)] * 3 + [_row(dom, 1024, v) for v in (9.0, 10.0, 11.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_csv(fp, fetch)
    _write_csv(wp, write)
    s = bench.summarize_pmc(str(fp), str(wp), 4, str(out))
    assert s["counters"]["FETCH_SIZE"]["scale"] == 2.0
    assert s["counters"]["WRITE_SIZE"]["scale"] == 1.0
    assert s["counters"]["FETCH_SIZE"]["launches"] == 3
    assert s["traffic_bytes_per_launch"] == round((100.0 * 2.0 + 10.0 * 1.0) * 1024)
    assert s["kernel_source_sha256"] == bench.kernel_source_hash()
    assert json.load(open(out)) == s


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    p = tmp_path / "t.json"
    json.dump({"traffic_bytes_per_launch": 123,
               "kernel_source_sha256": bench.kernel_source_hash()}, open(p, "w"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic() == 123
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
