"""Build libpagedkv.so (all HIP sources under csrc/) for gfx950, in place.

    python -m paged_kv_cache_tables_amd.build

Every source is compiled by hipcc for --offload-arch=gfx950 with packed-FP32
instruction generation disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpagedkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = True, extra_flags=()) -> str:
    srcs = sources()
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *srcs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
