"""Build libpagedkv.so (all HIP sources under csrc/) for gfx950, in place.

    python -m paged_kv_cache_tables_amd.build

Every source is compiled by hipcc for --offload-arch=gfx950 with packed-FP32
instruction generation disabled, one object per source (in parallel, under
_build/), then linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpagedkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


def build(verbose: bool = True, extra_flags=(), jobs: int = 0) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    srcs = sources()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    cmds, objs = [], []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra_flags, *inc, "-c", src, "-o", obj])
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    _run(link, verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
