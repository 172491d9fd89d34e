"""bench.py's host-side contract without a GPU: more than one GPU is refused
with a message (the path has no multi-GPU leg), a non-prefill workload name
is refused, and the traffic figure is reported only for the kernel source the
counters were taken on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    """The hash covers the kernel source and the headers it includes (found
    through its #include lines, recursively): a change to either makes the
    stored traffic figure stale; a header it does not include does not."""
    import bench
    from transformer_attention_diffattn_amd import traffic_summary as ts

    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    pkg = tmp_path / "transformer_attention_diffattn_amd"
    csrc = pkg / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text('#include "a.h"\nkernel source\n')
    (csrc / "a.h").write_text('#include "b.h"\nhelper\n')
    (csrc / "b.h").write_text("nested helper\n")
    (csrc / "other.h").write_text("not included\n")
    monkeypatch.setattr(ts, "PKG", str(pkg))
    h = ts.source_hash("k.hip")
    (prof / "x_traffic.json").write_text(json.dumps({"bytes_per_launch": 123, "source_sha256_16": h}))
    assert bench._traffic("x", "k.hip") == 123
    (csrc / "other.h").write_text("changed, still not included\n")
    assert bench._traffic("x", "k.hip") == 123
    (csrc / "b.h").write_text("changed nested helper\n")
    assert bench._traffic("x", "k.hip") is None
    (csrc / "b.h").write_text("nested helper\n")
    assert bench._traffic("x", "k.hip") == 123
    (csrc / "k.hip").write_text('#include "a.h"\nchanged kernel source\n')
    assert bench._traffic("x", "k.hip") is None
    assert bench._traffic("missing", "k.hip") is None
