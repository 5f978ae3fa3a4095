"""Build libssd.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m ssd_scan_amd.build   (or ssd_scan_amd.build.build())
Objects go to _build/ at the repository root; the shared library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libssd.so")
ARCH = "gfx950"

SOURCES = ["ssd_api.hip", "ssd_bwd.hip", "ssd_chunked.hip", "ssd_fused.hip", "ssd_step.hip",
           "ssd_stream.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-strict-aliasing",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# per-source flags: the stream kernel is scheduled for instruction-level
# parallelism (measured 1-2 % faster on the 2.7B-shaped layer than the default
# occupancy-driven schedule; its occupancy is fixed by LDS at one workgroup per CU)
SOURCE_FLAGS = {"ssd_stream.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link libssd.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
