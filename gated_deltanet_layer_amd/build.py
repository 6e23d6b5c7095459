"""Build libgdn.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Each source compiles to its own object (in parallel, under ``_build/`` at the
repository root), then one hipcc call links the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build", "obj")
SOURCES = ["gdn_api.cpp", "recurrent_step.hip", "chunk_fwd.hip", "chunk_fwd_ws.hip", "chunk_fwd_seg.hip",
           "chunk_fwd_wsc.hip", "recurrent_multi.hip", "chunk_bwd.hip",
           "prologue.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code (the host pass warns that it
    # does not know the feature; that is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", "-x", "hip", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libgdn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
