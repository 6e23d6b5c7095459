"""Build libgdn.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "recurrent_step.hip", "chunk_fwd.hip", "chunk_fwd_ws.hip", "chunk_fwd_wsc.hip", "recurrent_multi.hip", "chunk_bwd.hip", "prologue.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions in device code (the host pass warns that it
    # does not know the feature; that is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        srcs += (["-x", "hip", path] if s.endswith(".cpp") else [path])
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libgdn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
