"""Build libprism.so (gfx950 HIP kernels + C ABI) in the package directory.

    python -m dynamic_block_sparse_shape_amd.build

Each .hip source compiles to its own object (in parallel), then one shared
library is linked.  The objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libprism.so")
OBJDIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("PRISM_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.hip", "zone_shapes.hip", "pool_proxy.hip", "select.hip",
           "pairing.hip", "attn_fwd.hip", "attn_bwd.hip", "dropped.hip",
           "bridge.hip", "route.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is
    # expected, anything else is shown
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip()
                    and "is not a recognized feature" not in l)
    if err and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libprism.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []

    def one(src):
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        _run([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as pool:
        objs = list(pool.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
