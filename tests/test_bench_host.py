"""bench.py host logic on the CPU: the one-GPU contract, the HBM traffic record built from two
rocprofv3 counter runs (copy calibration, only the timed dispatches averaged), and the rule that
a committed traffic record is reported only for the launches it was taken over."""
import csv
import json
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_dir(path, kernel, values, copy_kib):
    """A rocprofv3 csv directory: `values` per dispatch of `kernel` (KiB), dispatch ids in
    order, then one large copy kernel whose counter reads `copy_kib`."""
    os.makedirs(path)
    rows = [{"Dispatch_Id": i + 1, "Kernel_Name": f"void kvc::{kernel}(kvc::DecodeArgs)",
             "Grid_Size": 65536, "Counter_Value": v} for i, v in enumerate(values)]
    rows.append({"Dispatch_Id": len(values) + 1, "Kernel_Name": "__amd_rocclr_copyBuffer",
                 "Grid_Size": 1 << 20, "Counter_Value": copy_kib})
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_traffic_record_calibrates_and_averages_the_timed_launches(tmp_path):
    kernel = "decode_partial_kernel<true, 1, 128, true, 1, false>"
    steps, layers, warm = 2, 3, 1
    # warm-up dispatches read far more; only the last steps x layers count
    fetch = [1e6] * (warm * layers) + [100.0, 110.0, 120.0, 130.0, 140.0, 150.0]
    write = [5e5] * (warm * layers) + [10.0] * (steps * layers)
    gib_kib = (1 << 30) / 1024
    _counter_dir(str(tmp_path / "F"), kernel, fetch, gib_kib / 2)   # FETCH_SIZE counts half
    _counter_dir(str(tmp_path / "W"), kernel, write, gib_kib)
    line = {"steps": steps, "warmup": warm,
            "config": {"workload": "w", "layers": layers, "append": "fused"},
            "roofline": {"kernel_match": kernel, "algorithmic_bytes_per_launch": 250_000,
                         "kernel_source_sha256_16": "0" * 16}}
    log = tmp_path / "bench.log"
    log.write_text("[bench] setting up\n" + json.dumps(line) + "\n")
    rec = bench.pmc_summary(str(tmp_path / "F"), str(tmp_path / "W"), str(log))
    assert rec["dispatches_averaged"] == [6, 6]
    assert abs(rec["fetch_scale"] - 2.0) < 1e-9 and abs(rec["write_scale"] - 1.0) < 1e-9
    assert rec["fetch_bytes"] == int(125.0 * 1024 * 2)
    assert rec["write_bytes"] == int(10.0 * 1024)
    assert rec["traffic_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert abs(rec["traffic_over_algorithmic"] - round((125.0 * 2048 + 10240) / 250_000, 4)) < 1e-9


def test_committed_traffic_is_reported_only_for_its_own_launches():
    w = workloads.LLAMA13B_PAGED
    rec = json.loads(open(bench.traffic_file(w)).readline())
    args = (rec["steps"], rec["warmup"], rec["layers"])
    current = rec["source_sha256_16"] == bench.source_hash(bench.workload_source(w))
    assert bench.measured_traffic(w, rec["append"], *args) == (
        rec["traffic_bytes"] if current else None)   # a record of another source is not used
    assert bench.measured_traffic(w, rec["append"], rec["steps"] + 1, *args[1:]) is None
    assert bench.measured_traffic(w, "separate", *args) is None
    assert bench.measured_traffic(workloads.TINY_GPT, "fused", *args) is None
