"""Build the HIP library in-tree: hipcc for gfx950 -> fully_sharded_amd/libfsdp_hip.so.

Run ``python -m fully_sharded_amd._build`` (or ``__graft_entry__.build()``).
It compiles every time it is called.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfsdp_hip.so")
SOURCES = ["plan.cpp", "kernels.hip", "abi.cpp", "graph.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# IEEE fp32: correctly rounded divide and sqrt, denormals kept, no fast-math,
# no implicit FMA contraction (the kernels write their FMAs explicitly), and
# no packed-fp32 instructions.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = True) -> str:
    objs = []
    os.makedirs(os.path.join(PKG, "_build"), exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(PKG, "_build", src + ".o")
        cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
