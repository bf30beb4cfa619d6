"""Build libbnn.so (the gfx950 HIP kernels and their C ABI) with hipcc, and
libbnn_calib.so (the VALU issue-rate probes the benchmark runs for its
roofline; not part of the product library).

Run as ``python -m xnor_popcount_gemm_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The libraries are built in-tree, next to this file.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbnn.so")
CALIB_SRCS = [os.path.join(HERE, "calib", "valu_rate.hip"), os.path.join(HERE, "calib", "hbm_stream.hip")]
CALIB_LIB = os.path.join(HERE, "libbnn_calib.so")
ARCH = "gfx950"


def hipcc() -> str:
    cand = [os.environ.get("HIPCC", ""), "/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""]
    for c in cand:
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbnn)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",                     # alpha*D and +R stay two rounded ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wall",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n if n > 0 else (os.cpu_count() or 1), 16))


def build_calib(verbose: bool = False) -> str:
    """Compile the issue-rate probes into libbnn_calib.so."""
    tmp = CALIB_LIB + ".tmp"
    cmd = [hipcc()] + [f for f in flags() if not f.startswith("-I")] + ["-shared"] + CALIB_SRCS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    sys.stderr.write(r.stderr)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, f"hipcc {' '.join(CALIB_SRCS)}", r.stdout, r.stderr)
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


# Per-source flags.  dense.hip: MFMA results in VGPRs (the VGPR form of
# v_mfma_f64_16x16x4_f64).  Left to choose, the compiler kept the fp64 first
# layer's loop-carried accumulators in VGPRs but let the MFMAs write AGPRs,
# and copied all 64 accumulator registers across and back every K chunk
# (4 VALU ops per MFMA in a loop of 32 MFMAs).
FILE_FLAGS = {"dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link libbnn.so;
    then build the probe library."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="bnn_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(so):
            src, obj = so
            cmd = [cc] + flags() + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            results = list(pool.map(compile_one, zip(srcs, objs)))
        for src, r in zip(srcs, results):
            sys.stderr.write(r.stderr)
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, f"hipcc -c {src}", r.stdout, r.stderr)
        tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_calib(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
