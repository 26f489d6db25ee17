"""Builds libfsdpshard.so in-tree with hipcc for gfx950.

The host indexer (csrc/unit.cpp) is plain C++; the kernels and the device
entry points (csrc/kernels.hip) are HIP. Flags that fix the numerics:
-ffp-contract=off (no fused multiply-add anywhere on the path), the default
correctly rounded fp32 division and square root (never -ffast-math), and
packed-fp32 instructions disabled for device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfsdpshard.so"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-mcode-object-version=5",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    noise = "is not a recognized feature for this target"
    rest = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if verbose and rest.strip():
        print(rest)


def build(out_dir: str | None = None, defines=(), verbose: bool = False) -> str:
    """Compiles the library; returns the path of the .so."""
    out_dir = out_dir or PKG
    obj_dir = os.path.join(out_dir, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    unit_o = os.path.join(obj_dir, "unit.o")
    kern_o = os.path.join(obj_dir, "kernels.o")
    _run([HIPCC, "-x", "c++", *COMMON, *dflags, "-c", os.path.join(CSRC, "unit.cpp"),
          "-o", unit_o], verbose)
    _run([HIPCC, "-x", "hip", *DEVICE, *COMMON, *dflags, "-c",
          os.path.join(CSRC, "kernels.hip"), "-o", kern_o], verbose)
    tmp = os.path.join(out_dir, LIB_NAME + ".tmp")
    _run([HIPCC, *DEVICE, "-shared", "-fPIC", "-o", tmp, unit_o, kern_o], verbose)
    final = os.path.join(out_dir, LIB_NAME)
    os.replace(tmp, final)
    shutil.rmtree(obj_dir, ignore_errors=True)
    return final


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
