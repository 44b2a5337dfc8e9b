"""The workgroup -> tile placement and the prefetch workgroups' roles (bigemm_tilemap.h, the
same host/device functions the kernels call), built with hipcc for the host and checked on the
CPU by tests/tilemap/tilemap_check.hip: every tile covered once, padding exactly when the
tiles fill at most half of the CUs and K is long, each XCD's prefetch workgroups indexed
0 .. nh - 1 once each, and each XCD's units exactly the distinct tile rows and columns of its
tiles."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_tile_map_and_prefetch_units(tmp_path):
    exe = str(tmp_path / "tilemap_check")
    src = os.path.join(ROOT, "tests", "tilemap", "tilemap_check.hip")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", src, "-o", exe], check=True,
                   capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert "tilemap ok" in r.stdout
