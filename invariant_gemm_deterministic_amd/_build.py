"""Build libbigemm.so (the gfx950 kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbigemm.so")
SOURCES = [os.path.join(CSRC, "bigemm_kernels.hip"), os.path.join(CSRC, "bigemm_rmsnorm.hip"),
           os.path.join(CSRC, "bigemm_attention.hip"),
           os.path.join(CSRC, "bigemm_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 ops are disabled for every HIP translation unit.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
