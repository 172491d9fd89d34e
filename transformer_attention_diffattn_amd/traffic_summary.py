"""Per-launch HBM traffic of one kernel from two rocprofv3 counter passes.

    python -m transformer_attention_diffattn_amd.traffic_summary \\
        --fetch <dir>/FETCH_SIZE/run_counter_collection.csv \\
        --write <dir>/WRITE_SIZE/run_counter_collection.csv \\
        --kernel prefill_bf16_kernel --name prefill_layer1p4b \\
        --workload layer1p4b_bf16_b4h16n2048d64 --source prefill.hip \\
        --calib-mib 1024 --algorithmic 134217728 > profiles/prefill_layer1p4b_traffic.json

``--kernel`` may be given more than once (a step of several kernels, such as
decode's split and merge kernels): the figure is then the sum of each
kernel's per-dispatch mean.

The passes are runs of ``bench.py ... --copy-calib-mib M``, which also makes
one device copy of M MiB.  FETCH_SIZE and WRITE_SIZE are in KiB per dispatch;
each is scaled by the factor that makes the copy read and write exactly M MiB
(the counters' own unit and sampling), then averaged over the kernel's
dispatches.  The source hash (the kernel source and the headers it includes)
lets ``bench.py`` report the figure only while the kernel is the one the
counters were taken on.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))


def _with_includes(path: str, seen: list) -> list:
    """path and every header it includes with #include "..." (resolved next
    to the including file), depth first, each once."""
    path = os.path.normpath(path)
    if path in seen:
        return seen
    seen.append(path)
    with open(path) as fh:
        for line in fh:
            m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
            if m:
                _with_includes(os.path.join(os.path.dirname(path), m.group(1)), seen)
    return seen


def source_hash(sources: str) -> str:
    """Hash of the kernel sources (comma-separated names under csrc/) together
    with the headers they include: a counter profile is current only while
    this hash is unchanged."""
    files: list = []
    for n in sources.split(","):
        _with_includes(os.path.join(PKG, "csrc", n), files)
    h = hashlib.sha256()
    for path in files:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, pattern: str) -> list:
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if pattern in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return vals


def _copy_value(path: str) -> float:
    """Counter value of the calibration copy: the largest dispatch of the
    runtime's copy kernel in the pass."""
    best = 0.0
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "copyBuffer" in name or "elementwise_kernel" in name and "copy" in name.lower():
                best = max(best, float(r["Counter_Value"]))
    return best


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--kernel", required=True, action="append", help="substring of a kernel name (repeatable)")
    ap.add_argument("--name", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--source", required=True, help="csrc file(s) the kernel is built from, comma separated")
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--algorithmic", type=int, required=True, help="algorithmic bytes per launch")
    a = ap.parse_args()
    fetch_kib = write_kib = 0.0
    counts = []
    for k in a.kernel:
        f = _per_dispatch(a.fetch, k)
        w = _per_dispatch(a.write, k)
        if not f or not w:
            raise SystemExit(f"no dispatch of {k!r} in the counter files")
        fetch_kib += sum(f) / len(f)
        write_kib += sum(w) / len(w)
        counts.append(len(f))
    calib_kib = a.calib_mib * 1024.0
    cf, cw = _copy_value(a.fetch), _copy_value(a.write)
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration copy found in the counter files")
    ff, fw = calib_kib / cf, calib_kib / cw
    fetch_b, write_b = fetch_kib * ff * 1024, write_kib * fw * 1024
    out = {
        "kernel": " + ".join(a.kernel), "workload": a.workload, "dispatches": min(counts),
        "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
        "fetch_factor": ff, "write_factor": fw,
        "bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes": int(round(fetch_b)), "write_bytes": int(round(write_b)),
        "algorithmic_bytes": a.algorithmic,
        "source_sha256_16": source_hash(a.source),
    }
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
