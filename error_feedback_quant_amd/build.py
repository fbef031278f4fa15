"""Build libecho.so (gfx950) from csrc/ with hipcc, in-tree.

Flags: -ffp-contract=off keeps every a*b+c as two rounded operations (the
results must match the CPU definition bit for bit); packed fp32 instructions
are disabled; fp32 denormals are kept (no flush to zero).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libecho.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, "echo_api.hip")]


# test-only device code: the kernels' helpers evaluated on their own, built
# with the library's flags (loaded by tests/test_gpu_*.py only)
CHECK_SRC = os.path.join(ROOT, "tests", "c", "recip_scale_check.hip")
CHECK_LIB = os.path.join(ROOT, "tests", "c", "librecip_scale_check.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if noise not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {LIB}")
    if msgs and verbose:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    build_check(verbose)
    return LIB


def build_check(verbose: bool = False) -> str:
    tmp = CHECK_LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", CSRC, CHECK_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stderr or "").splitlines() if "is not a recognized feature for this target" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {CHECK_LIB}")
    os.replace(tmp, CHECK_LIB)
    return CHECK_LIB


if __name__ == "__main__":
    print(build(verbose=True))
