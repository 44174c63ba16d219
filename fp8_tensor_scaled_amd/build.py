"""Build the HIP library libfp8lin.so for gfx950 (in-tree, next to this file).

Usage: python -m fp8_tensor_scaled_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8lin.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemm_tiled.hip", "gemm_skinny.hip"]
# the benchmark's ceiling kernels, a library of their own that only bench.py loads
BENCH_LIB = os.path.join(HERE, "libfp8bench.so")
BENCH_SOURCES = ["bench_ref.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8lin.so)")


def _flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Wno-unused-function",
        # keep hipcc from forming packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep single-lane atomics as written: the atomic optimizer turns
        # them into wave-wide reductions that read the returned value at
        # once, so the quantize fold's round trips would block the stores
        # issued after them
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfp8lin.so (and the
    benchmark's reference kernels, libfp8bench.so); returns the library's
    path."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES) + len(BENCH_SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES + BENCH_SOURCES))
    for lib, parts in ((LIB, objs[:len(SOURCES)]), (BENCH_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
