"""Build the gfx950 HIP library libqgemm.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemm.so")

SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "gemm_i8_wide.hip", "gemm_mx_dma.hip", "gemm_w4a8.hip",
           "unpack.hip", "ceiling.hip"]
OBJDIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-fast-math",
    "-ffp-contract=off",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-Wl,-rpath,/opt/rocm/lib",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build_library(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared
    library; every call compiles everything again."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJDIR, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f not in ("-shared",) and not f.startswith("-Wl,")]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [hipcc(), *compile_flags, "-c", "-I", os.path.join(ROOT, "include"),
                           os.path.join(CSRC, src), "-o", obj]))

    def run(job):
        obj, cmd = job
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(run, jobs))
    failed = [(o, r) for o, r in results if r.returncode != 0]
    for _, r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed compiling " + ", ".join(os.path.basename(o) for o, _ in failed))
    tmp = LIB + ".tmp"
    link = [hipcc(), *HIPCC_FLAGS, *[o for o, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libqgemm.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
