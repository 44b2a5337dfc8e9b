"""Build and load the device negative control (test infrastructure only)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nc4.hip")
LIB = os.path.join(HERE, "libnc4.so")


def build() -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fvisibility=hidden",
                    SRC, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.nc4_gemm_bf16.restype = ctypes.c_int
    lib.nc4_gemm_bf16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    return lib
