"""Build libbnn.so (the gfx950 HIP kernels and their C ABI) with hipcc.

Run as ``python -m xnor_popcount_gemm_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbnn.so")
ARCH = "gfx950"


def hipcc() -> str:
    cand = [os.environ.get("HIPCC", ""), "/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""]
    for c in cand:
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbnn)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",                     # alpha*D and +R stay two rounded ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wall",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
