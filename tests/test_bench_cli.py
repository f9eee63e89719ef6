"""Host-side checks of bench.py: the single-GPU guard and the HBM-traffic
calibration (FETCH_SIZE / WRITE_SIZE scaled by a copy of known size)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, **kw):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          cwd=ROOT, timeout=300, **kw)


def test_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_refuses_a_distributed_launch():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run([], env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr


def _counter_dir(tmp_path, name, counter, rows):
    d = tmp_path / name / "host" / "pid"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})
    return str(tmp_path / name)


def test_traffic_calibration(tmp_path):
    k = "void mta::v4::mta_fwd_v4<6, 11, false, false>(mta::Params, mta::v4::PrepArgs)"
    fetch = _counter_dir(tmp_path, "fetch", "FETCH_SIZE", [(k, 100.0), (k, 300.0), ("other", 1e9)])
    write = _counter_dir(tmp_path, "write", "WRITE_SIZE", [(k, 50.0), (k, 50.0)])
    # a 512 MiB copy that the fetch counter reports at half its size, the write counter in full
    copyf = _counter_dir(tmp_path, "copyF", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 262144.0)])
    copyw = _counter_dir(tmp_path, "copyW", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 524288.0)])
    out = tmp_path / "traffic.json"
    r = _run(["--config", "needle4k", "--copy-mb", "512", "--traffic-file", str(out), "--summarize-pmc", fetch, write,
              copyf, copyw])
    assert r.returncode == 0, r.stderr
    e = json.load(open(out))["needle4k"]
    assert e["dispatches"] == 2
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["read_bytes"] == 200 * 2 * 1024
    assert e["write_bytes"] == 50 * 1024
    assert e["bytes_per_launch"] == e["read_bytes"] + e["write_bytes"]
    assert len(e["sources"]) == 16
