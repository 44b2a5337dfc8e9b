"""Batch invariance on the GPU, byte for byte (GPU outputs compared only with GPU
outputs), through the C ABI. Workloads and cells: see tests/harness.py."""
import json
import os

import numpy as np
import pytest
import torch

import harness as H
from bigemm_inputs import (SEED_W, SEED_X, normal_bf16, linspace_bf16, normal_e4m3, e8m0_scales,
                           e8m0_kvar_scales, SCALE_SEED_OFFSET)
from gpu_util import DEV, GpuGemm, dev_bf16, dev_u8, require_gpu, rows_alone, run

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _mboundaries():
    with open(os.path.join(GOLDEN, "m_boundaries.txt")) as f:
        return [int(v) for ln in f if not ln.startswith("#") for v in ln.split()]


def _ab_rows(M):
    """Target rows 0, mid, last (not deduplicated: 3 cells per M)."""
    return [0, M // 2, M - 1]


# ------------------------------------------------------------ small bf16 workload
def test_small_bf16_ab_cells():
    """X[M,256] . W[256,128], N(0,1), M in {1,4,8,16,32}: 15 A/B cells."""
    gemm = GpuGemm()
    W = (normal_bf16(SEED_W, (256, 128)),)
    make = H.rows_bf16(256)
    cells = [H.ab_cell(gemm, make, W, M, r) for M in (1, 4, 8, 16, 32) for r in _ab_rows(M)]
    H.report("bf16 X[M,256].W[256,128]", cells, K=256, N=128, dtype="bf16")
    assert len(cells) == 15
    bad = [c for c in cells if c["ab"] or c["canon"]]
    assert not bad, bad


def test_small_bf16_position_and_repeat():
    gemm = GpuGemm()
    W = (normal_bf16(SEED_W, (256, 128)),)
    make = H.rows_bf16(256)
    for M in (2, 4, 8, 16, 32, 129, 300):
        d = H.position_cell(gemm, make, W, M)
        assert all(v == 0 for v in d.values()), (M, d)
    assert H.repeat_cell(gemm, make(SEED_X, 32), W, n=5) == 0


# --------------------------------------------------------------- linspace workload
def test_linspace_row0_prefix_vs_batch():
    """bytes((a[:1] . b)[0]) == bytes((a . b)[0]); also rows mid and last alone vs in batch."""
    B, D = 2048, 4096
    ad = dev_bf16(linspace_bf16(-1000.0, 1000.0, B * D, (B, D)))
    bd = dev_bf16(linspace_bf16(-1000.0, 1000.0, D * D, (D, D)))
    Y = run((ad,), (bd,))
    alone = rows_alone((ad,), (bd,), [0, B // 2, B - 1])
    for r, y in zip([0, B // 2, B - 1], alone):
        assert H.byte_diff(y, Y[r]) == 0, r


def test_linspace_vendor_contrast(capsys):
    """Informative contrast, not a requirement: the vendor GEMM (torch.mm through
    hipBLASLt, bf16 in and out) on the same experiment. Its row 0 alone and in the
    batch are allowed to differ (its kernel choice follows the shape); the number of
    differing bytes is printed. Ours is 0 for the same row."""
    import torch
    B, D = 2048, 4096
    a = dev_bf16(linspace_bf16(-1000.0, 1000.0, B * D, (B, D))).view(torch.bfloat16)
    b = dev_bf16(linspace_bf16(-1000.0, 1000.0, D * D, (D, D))).view(torch.bfloat16)
    vendor = H.byte_diff(torch.mm(a[:1], b)[0], torch.mm(a, b)[0])
    ours = H.byte_diff(run((a[:1].view(torch.int16),), (b.view(torch.int16),))[0],
                       run((a.view(torch.int16),), (b.view(torch.int16),))[0])
    torch.cuda.synchronize()
    with capsys.disabled():
        print(f"\n  linspace row 0, alone vs in the batch of {B}: torch.mm {vendor} differing bytes, bigemm {ours}")
    assert ours == 0


# ------------------------------------------------------ projection workload (M sweep)
@pytest.mark.parametrize("N", [4096, 14336])
def test_projection_msweep(N):
    """X_full[4096,4096] ~ N(0,1), W[4096,N] ~ N(0,0.02); every row of every prefix
    X[:M] equals that row of the M=4096 result, M across tile and wave boundaries."""
    K = 4096
    xd = dev_bf16(normal_bf16(SEED_X, (4096, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N), 0.02))
    Yfull = run((xd,), (wd,))
    Ms = sorted(set(_mboundaries() + [512, 1024, 2048, 4095, 4096]))
    out = torch.empty_like(Yfull)
    bad = {}
    for M in Ms:
        YM = run((xd[:M],), (wd,), out=out[:M])
        d = H.byte_diff(YM, Yfull[:M])
        for r, y in zip(H.row_positions(M), rows_alone((xd,), (wd,), H.row_positions(M))):
            d += H.byte_diff(y, Yfull[r])
        if d:
            bad[M] = d
    assert not bad, bad


def test_projection_repeat_and_streams():
    """Repeated calls and calls on two streams at once give identical bytes."""
    M = K = N = 4096
    xd = dev_bf16(normal_bf16(SEED_X, (M, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N), 0.02))
    Y0 = run((xd,), (wd,))
    for _ in range(3):
        assert H.byte_diff(run((xd,), (wd,)), Y0) == 0
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    y1, y2 = torch.empty_like(Y0), torch.empty_like(Y0)
    torch.cuda.synchronize()
    import invariant_gemm_deterministic_amd as bg
    with torch.cuda.stream(s1):
        bg.mm(xd, wd, out=y1)
    with torch.cuda.stream(s2):
        bg.mm(xd, wd, out=y2)
    torch.cuda.synchronize()
    assert H.byte_diff(y1, Y0) == 0 and H.byte_diff(y2, Y0) == 0


# ------------------------------------------------------------ long-K workload
def test_long_k_invariance():
    """[1024,16384] . [16384,1024], N(0,1): M in {1, 64, 1024}, rows vs M=1024."""
    M, K, N = 1024, 16384, 1024
    xd = dev_bf16(normal_bf16(SEED_X, (M, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N)))
    Y = run((xd,), (wd,))
    for m in (1, 64, 1024):
        assert H.byte_diff(run((xd[:m],), (wd,)), Y[:m]) == 0, m
    for r, y in zip([0, 512, 1023], rows_alone((xd,), (wd,), [0, 512, 1023])):
        assert H.byte_diff(y, Y[r]) == 0, r


# -------------------------------------------------------------------- MXFP8 grid
def _grid():
    with open(os.path.join(GOLDEN, "bi_cell_grid.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("combo", [("ID", "ID"), ("ID", "VAR"), ("VAR", "ID"), ("VAR", "VAR")],
                         ids=lambda c: f"{c[0]}-{c[1]}")
def test_mxfp8_ab_grid(combo):
    """The issue's matrix: M in {1..64}, K in {128..2048}, N in {64..512}, target rows
    {0, mid, last}: 360 A/B cells per scale combination (1440 in all)."""
    g = _grid()
    xk, wk = combo[0].lower(), combo[1].lower()
    gemm = GpuGemm()
    n = 0
    bad = []
    for K in g["K"]:
        make = H.rows_mx(K, xk)
        for N in g["N"]:
            W = (normal_e4m3(SEED_W, (K, N)), e8m0_scales(SEED_W + SCALE_SEED_OFFSET, (K // 32, N), wk))
            for M in g["M_per_rank"]:
                for r in _ab_rows(M):
                    c = H.ab_cell(gemm, make, W, M, r)
                    H.report(f"MXFP8 {combo[0]},{combo[1]}", [c], K=K, N=N, dtype="e4m3")
                    n += 1
                    if c["ab"] or c["canon"]:
                        bad.append((K, N, c))
    assert n == 360
    assert not bad, bad[:5]


def test_mxfp8_position_and_kvar():
    """Position cells, and scales that vary along K only (same for every row)."""
    gemm = GpuGemm()
    for kind in ("var", "kvar"):
        K, N = 1024, 256
        wk = "var" if kind == "var" else "kvar"
        if wk == "kvar":
            WS = e8m0_kvar_scales(SEED_W + SCALE_SEED_OFFSET, K // 32, N, k_axis=0)
        else:
            WS = e8m0_scales(SEED_W + SCALE_SEED_OFFSET, (K // 32, N), "var")
        W = (normal_e4m3(SEED_W, (K, N)), WS)
        make = H.rows_mx(K, kind)
        for M in (2, 17, 64, 129, 300):
            d = H.position_cell(gemm, make, W, M)
            assert all(v == 0 for v in d.values()), (kind, M, d)


def test_mxfp8_msweep():
    K, N = 2048, 512
    xd = (dev_u8(normal_e4m3(SEED_X, (1024, K))), dev_u8(e8m0_scales(SEED_X + 100, (1024, K // 32), "var")))
    wd = (dev_u8(normal_e4m3(SEED_W, (K, N))), dev_u8(e8m0_scales(SEED_W + 100, (K // 32, N), "var")))
    Y = run(xd, wd)
    for M in _mboundaries() + [1024]:
        assert H.byte_diff(run(tuple(a[:M] for a in xd), wd), Y[:M]) == 0, M


# ------------------------------------------------------ device negative control
def test_nc4_device_split_k_is_caught():
    """The M sweep on the GPU is not vacuous: a device GEMM whose K split depends on
    M (tests/nc4) shows byte diffs across the 64-row boundaries at the projection
    magnitudes, while libbigemm shows none on the same inputs."""
    import ctypes
    import nc4
    lib = nc4.load()
    K, N, Mmax = 4096, 128, 256
    xd = dev_bf16(normal_bf16(SEED_X, (Mmax, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N), 0.02))
    stream = torch.cuda.current_stream().cuda_stream

    def nc4_run(m):
        y = torch.empty((m, N), dtype=torch.float32, device=DEV)
        assert lib.nc4_gemm_bf16(m, N, K, xd.data_ptr(), K, wd.data_ptr(), N, y.data_ptr(), N, stream) == 0
        torch.cuda.synchronize()
        return y

    Yn = nc4_run(Mmax)
    Yb = run((xd,), (wd,))
    caught = {}
    for M in _mboundaries():
        assert H.byte_diff(run((xd[:M],), (wd,)), Yb[:M]) == 0, M
        caught[M] = H.byte_diff(nc4_run(M), Yn[:M])
    assert caught[256] == 0 and caught[193] == 0, caught          # same split count as the full batch
    assert all(caught[M] > 0 for M in (1, 64, 65, 128, 129, 192)), caught
    assert H.byte_diff(nc4_run(64), nc4_run(64)) == 0             # deterministic run to run
