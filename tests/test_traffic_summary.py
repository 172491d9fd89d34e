"""The per-launch traffic figure computed from counter files (host logic only)."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scaled_by_the_calibration_copy(tmp_path):
    # the copy of 1 MiB reads as 512 KiB fetched (factor 2) and 1024 KiB written (factor 1)
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    k = "void diffattn::prefill_bf16_kernel<64, true, true>(diffattn::PrefillArgs)"
    _write(fetch, [(k, "FETCH_SIZE", 100.0), (k, "FETCH_SIZE", 300.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0),
                   ("other", "FETCH_SIZE", 9999.0)])
    _write(write, [(k, "WRITE_SIZE", 50.0), (k, "WRITE_SIZE", 50.0), ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    out = subprocess.run(
        [sys.executable, "-m", "transformer_attention_diffattn_amd.traffic_summary", "--fetch", str(fetch),
         "--write", str(write), "--kernel", "prefill_bf16_kernel<64, true, true>", "--name", "x", "--workload", "y",
         "--source", "prefill.hip", "--calib-mib", "1", "--algorithmic", "1000"],
        capture_output=True, text=True, check=True, cwd=ROOT).stdout
    t = json.loads(out)
    assert t["dispatches"] == 2
    assert t["fetch_factor"] == 2.0 and t["write_factor"] == 1.0
    assert t["fetch_bytes"] == 200 * 2 * 1024  # mean 200 KiB, scaled by 2
    assert t["write_bytes"] == 50 * 1024
    assert t["bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    assert len(t["source_sha256_16"]) == 16


def test_traffic_of_a_two_kernel_step(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fetch, [("split_kernel<x>", "FETCH_SIZE", 1000.0), ("merge_kernel<x>", "FETCH_SIZE", 10.0),
                   ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1024.0)])
    _write(write, [("split_kernel<x>", "WRITE_SIZE", 100.0), ("merge_kernel<x>", "WRITE_SIZE", 1.0),
                   ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    out = subprocess.run(
        [sys.executable, "-m", "transformer_attention_diffattn_amd.traffic_summary", "--fetch", str(fetch),
         "--write", str(write), "--kernel", "split_kernel", "--kernel", "merge_kernel", "--name", "x",
         "--workload", "y", "--source", "decode.hip", "--calib-mib", "1", "--algorithmic", "1"],
        capture_output=True, text=True, check=True, cwd=ROOT).stdout
    t = json.loads(out)
    assert t["fetch_bytes"] == 1010 * 1024 and t["write_bytes"] == 101 * 1024
    assert t["kernel"] == "split_kernel + merge_kernel"
