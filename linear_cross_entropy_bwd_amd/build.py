"""Build the HIP library ``libflce.so`` in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc for ``--offload-arch=gfx950``
and the host-only ``csrc/*.cpp`` files as C++; all objects link into
``linear_cross_entropy_bwd_amd/libflce.so``.  Run as
``python -m linear_cross_entropy_bwd_amd.build`` or through
``__graft_entry__.build()``.
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
BUILD = os.path.join(ROOT, "_build", "flce")
LIB = os.path.join(PKG, "libflce.so")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Keep the compiler from forming packed fp32 arithmetic in device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [_hipcc(), "-x", "hip", *COMMON, *DEVICE, "-c", src, "-o", obj]
    else:
        cmd = [_hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libflce.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    jobs = min(8, len(srcs), max(1, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
