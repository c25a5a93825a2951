"""Host-side logic of bench.py, on the CPU: the counter-traffic summary (each
counter scaled by what it reads for a copy of known size), the guard that
reports counter figures only for the workload, shape and kernel sources they were
taken on, the cache rotation of one-layer workloads, and the one-GPU refusal."""
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


SHAPE = {"B": 1, "h_q": 32, "h_k": 4, "h_v": 16, "d": 64, "l_kv": 131072, "N": 512, "R": 16,
         "caches": 16}


def test_summarize_pmc_scales_each_counter_by_the_copy(tmp_path):
    sel = "void saga::k_select<64, 1, false, 4>(saga::SelectArgs)"
    att = "void saga::k_attend<64, 15, false>(saga::AttendArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # a 4 MiB copy: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them; small
    # copies (below a quarter of the known size) and other kernels are ignored
    fetch = [_row(copy, 1, 2048.0)] * 3 + [_row(copy, 1, 16.0)] + \
        [_row(sel, 1024, v) for v in (99.0, 100.0, 101.0)] + [_row(att, 128, 7.0)] * 2 + \
        [_row("other", 8, 1e9)]
    write = [_row(copy, 1, 4096.0)] * 3 + [_row(sel, 1024, v) for v in (9.0, 10.0, 11.0)] + \
        [_row(att, 128, 1.0)] * 2
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_csv(fp, fetch)
    _write_csv(wp, write)
    s = bench.summarize_pmc(str(fp), str(wp), 4, str(out), "wl", SHAPE)
    assert s["scales"]["FETCH_SIZE"]["scale"] == 2.0
    assert s["scales"]["WRITE_SIZE"]["scale"] == 1.0
    assert s["dominant"] == "saga::k_select<64, 1, false, 4>"
    k = s["kernels"]
    assert k["saga::k_select<64, 1, false, 4>"]["FETCH_SIZE"]["launches"] == 3
    assert s["traffic_bytes_per_launch"] == round((100.0 * 2.0 + 10.0 * 1.0) * 1024)
    assert k["saga::k_attend<64, 15, false>"]["bytes_per_launch"] == round((7 * 2 + 1) * 1024)
    assert "other" not in k
    assert s["kernel_source_sha256"] == bench.kernel_source_hash()
    assert s["workload"] == "wl" and s["shape"] == SHAPE
    assert json.load(open(out)) == s


def test_traffic_is_keyed_on_workload_shape_and_sources(tmp_path, monkeypatch):
    """A counter summary is reported only for the workload, shape and kernel
    sources it was taken on (a run at another context length or config must not
    report the 128K figure)."""
    p = tmp_path / "t.json"
    json.dump({"traffic_bytes_per_launch": 123, "workload": "wl", "shape": SHAPE,
               "kernels": {}, "kernel_source_sha256": bench.kernel_source_hash()}, open(p, "w"))
    assert bench.measured_traffic("wl", SHAPE, str(p))["traffic_bytes_per_launch"] == 123
    assert bench.measured_traffic("other", SHAPE, str(p)) is None
    assert bench.measured_traffic("wl", dict(SHAPE, l_kv=32768), str(p)) is None
    assert bench.measured_traffic("wl", SHAPE, str(tmp_path / "missing.json")) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("wl", SHAPE, str(p)) is None


def test_one_layer_workloads_rotate_over_a_gib_of_keys():
    assert bench.rotation_caches(16, 64 << 20) == 16      # the 16-layer workload runs its layers
    assert bench.rotation_caches(1, 16 << 20) == 64       # Llama shape at 32K: 16 MiB of keys
    assert bench.rotation_caches(1, 128 << 20) == 8       # Qwen shape at 128K: 128 MiB
    assert bench.rotation_caches(1, 3 << 30) == 1
    assert bench.rotation_caches(1, 16 << 20, forced=1) == 1


def test_workload_names_carry_overrides_and_rotation():
    import argparse

    def args(**kw):
        a = dict(config="llama32-1b-128k-16L", B=0, l_kv=0, R=0, N=0, caches=0)
        a.update(kw)
        return argparse.Namespace(**a)

    cfg, ci, name, L, shape = bench.resolve_workload(args())
    assert name == "llama32-1b-128k-16L" and L == 16 and shape == SHAPE
    cfg, ci, name, L, shape = bench.resolve_workload(args(config="llama32-1b-32k"))
    assert name == "llama32-1b-32k caches=64" and L == 64 and shape["l_kv"] == 32768
    cfg, ci, name, L, shape = bench.resolve_workload(args(l_kv=4096, R=4))
    assert name == "llama32-1b-128k-16L l_kv=4096 R=4" and shape["R"] == 4
    assert bench.traffic_file(name).endswith("traffic_llama32-1b-128k-16L_l_kv4096_R4.json")
    cfg, ci, name, L, shape = bench.resolve_workload(args(B=4))
    assert name == "llama32-1b-128k-16L B=4" and shape["B"] == 4 and cfg.B == 4
    assert bench.resolve_workload(args(config="nope")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
