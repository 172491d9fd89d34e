"""Build libdiffattn.so (HIP, gfx950) in-tree with hipcc.

    python -m transformer_attention_diffattn_amd.build_lib

Sources are compiled in parallel into ``_build/`` at the repository root and
linked into ``transformer_attention_diffattn_amd/libdiffattn.so``.  Only the
symbols declared in ``include/diffattn.h`` are exported.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libdiffattn.so")
SOURCES = ["api.hip", "prefill.hip", "schedule.hip", "decode.hip", "backward.hip", "quant.hip", "proj.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                "-Wall", "-Wno-unused-function", "-I", INCLUDE]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass warns that it does not know the device-only feature
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(failed)}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
