"""Build librq.so (gfx950) in-tree with hipcc.

    python -m rotated_w4a4_quantized_amd.build      # or build() from Python

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled and no floating-point contraction (the rotations and quantizers are
pinned to explicit fp32/fp64 operation sequences).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librq.so")
SOURCES = ["rq_host.cpp", "rq_api.cpp", "rq_device.cpp", "rq_rpbh.hip", "rq_dense.hip",
           "rq_gemm_w4a4.hip", "rq_gemm_i8.hip", "rq_gemm_fp6.hip", "rq_gemm_codebook.hip",
           "rq_gemm_mx.hip", "rq_trdq.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wno-unused-function"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link librq.so; returns the
    library path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmds.append([HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
