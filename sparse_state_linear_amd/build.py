"""Build the gfx950 HIP library libsse_amd.so in-tree with hipcc.

Every .hip source is compiled to an object in parallel (one hipcc process
each), then the objects are linked into the shared library.  All HIP sources
are compiled with packed fp32 instructions disabled (the compiler would
otherwise fuse pairs of fp32 operations into v_pk_* forms).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsse_amd.so")
ARCH = os.environ.get("SSE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="sse_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(compile_one, zip(srcs, objs)))
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", out + ".tmp", *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
