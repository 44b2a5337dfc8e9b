"""The C ABI's host-side validation (bigemm_api.cpp) built for the CPU with the address and
undefined-behaviour sanitizers (g++, no GPU code: the kernel launchers are host stand-ins
that abort if reached) and driven over boundary and hostile arguments by
tests/sanitize/validators.cpp. Any signed overflow, out-of-bounds access or bad shift in the
validators aborts the program; it also checks bigemm_check_args against the header's rules."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_validators_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "validators")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "invariant_gemm_deterministic_amd", "csrc", "bigemm_api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "validators.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "validators ok" in r.stdout
