"""fp16 inputs, bf16 output and int8 inputs on the GPU, through the C ABI.

Parity: fp16 against the oracle's fp64 product within the fp32-accumulation
bound; bf16 output as exactly the round-to-nearest-even of the fp32 output of
the same call (and within the bound widened by one bf16 rounding); int8 equal
to the oracle's exact int64 product. Batch invariance: the same A/B, position
and M-sweep cells as the bf16 and MXFP8 tests, byte for byte.
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from bigemm_inputs import (SCALE_SEED_OFFSET, SEED_W, SEED_X, e8m0_scales, int_f16, int_i8, normal_bf16,
                           normal_e4m3, normal_f16)
from gpu_util import DEV, GpuGemm, dev_bf16, dev_u8, require_gpu, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def dev_f16(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)


def dev_i8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def rne_bf16_bits(y_f32: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bits, round to nearest even; a NaN keeps its top half with
    the quiet bit (bit 6) set — the rounding the header states for a bf16 output."""
    u = np.ascontiguousarray(y_f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------------- fp16
F16_SHAPES = [(1, 8, 8), (37, 200, 136), (130, 264, 200), (257, 128, 1024), (64, 520, 2048)]


@pytest.mark.parametrize("M,N,K", F16_SHAPES)
def test_f16_parity(M, N, K):
    X, W = normal_f16(51, (M, K)), normal_f16(52, (K, N))
    y = run((dev_f16(X),), (dev_f16(W),)).cpu().numpy()
    Y, S = oracle.gemm_f16(X, W)
    assert oracle.max_normalized_error(y, Y, S) <= oracle.PARITY_TOL


@pytest.mark.parametrize("M,N,K", [(5, 40, 24), (130, 264, 2048)])
def test_f16_integer_exact(M, N, K):
    """Integers in [-64, 64]: every partial sum is an exact integer below 2^24."""
    X, W = int_f16(53, (M, K), -64, 64), int_f16(54, (K, N), -64, 64)
    y = run((dev_f16(X),), (dev_f16(W),)).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), oracle.gemm_f16(X, W, want_s=False))


def test_f16_ab_and_position_cells():
    gemm = GpuGemm()
    W = (normal_f16(SEED_W, (256, 128)).view(np.float16),)
    make = H.rows_f16(256)
    cells = [H.ab_cell(gemm, make, W, M, r) for M in (1, 4, 8, 16, 32) for r in (0, M // 2, M - 1)]
    H.report("fp16 X[M,256].W[256,128]", cells, K=256, N=128, dtype="f16")
    assert not [c for c in cells if c["ab"] or c["canon"]]
    for M in (17, 129, 300):
        assert all(v == 0 for v in H.position_cell(gemm, make, W, M).values()), M


def test_f16_msweep():
    K, N = 1024, 512
    xd = dev_f16(normal_f16(SEED_X, (1024, K)))
    wd = dev_f16(normal_f16(SEED_W, (K, N), 0.05))
    Y = run((xd,), (wd,))
    for M in (1, 7, 64, 65, 128, 129, 193, 256, 1000):
        assert H.byte_diff(run((xd[:M],), (wd,)), Y[:M]) == 0, M


# ------------------------------------------------------------------ bf16 output
def _inputs(kind, M, N, K):
    if kind == "bf16":
        X, W = normal_bf16(61, (M, K)), normal_bf16(62, (K, N))
        return (dev_bf16(X),), (dev_bf16(W),), lambda: oracle.gemm_bf16(X, W)
    if kind == "f16":
        X, W = normal_f16(63, (M, K)), normal_f16(64, (K, N))
        return (dev_f16(X),), (dev_f16(W),), lambda: oracle.gemm_f16(X, W)
    X, W = normal_e4m3(65, (M, K)), normal_e4m3(66, (K, N))
    XS, WS = e8m0_scales(165, (M, K // 32), "var"), e8m0_scales(166, (K // 32, N), "var")
    return ((dev_u8(X), dev_u8(XS)), (dev_u8(W), dev_u8(WS)), lambda: oracle.gemm_mxfp8(X, W, XS, WS))


@pytest.mark.parametrize("kind", ["bf16", "f16", "mx"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (130, 272, 512), (257, 128, 1024)])
def test_bf16_output_is_the_rounded_f32_output(kind, M, N, K):
    xd, wd, _ = _inputs(kind, M, N, K)
    y32 = run(xd, wd).cpu().numpy()
    ybf = run(xd, wd, out_dtype=torch.bfloat16)
    assert ybf.dtype == torch.bfloat16
    assert np.array_equal(bf16_bits(ybf), rne_bf16_bits(y32))


@pytest.mark.parametrize("kind", ["bf16", "f16", "mx"])
def test_bf16_output_parity(kind):
    xd, wd, ref = _inputs(kind, 130, 272, 512)
    y = run(xd, wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    Y, S = ref()
    assert oracle.max_normalized_error(y, Y, S) <= oracle.PARITY_TOL_BF16_OUT


def test_bf16_output_special_values():
    """A NaN input row gives a NaN bf16 row; a row whose sums exceed the range gives
    inf; the other rows are the rounded fp32 values."""
    X = normal_bf16(67, (48, 64))
    W = np.full((64, 32), 0x3F80, np.uint16)   # 1.0: every partial sum has one sign per row
    X[3, 5] = 0x7FC0                            # bf16 NaN
    X[7, :] = 0x7E80                            # 2^126: row 7 sums to 2^132, beyond binary32
    xd, wd = (dev_bf16(X),), (dev_bf16(W),)
    y32 = run(xd, wd).cpu().numpy()
    ybf = bf16_bits(run(xd, wd, out_dtype=torch.bfloat16))
    assert np.array_equal(ybf, rne_bf16_bits(y32))
    assert np.isnan(y32[3]).all() and np.isposinf(y32[7]).all()
    assert (ybf[7] == 0x7F80).all()


def test_bf16_output_msweep_and_ab():
    K, N = 2048, 1024
    xd = dev_bf16(normal_bf16(SEED_X, (1024, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N), 0.02))
    Y = run((xd,), (wd,), out_dtype=torch.bfloat16)
    for M in (1, 8, 63, 64, 65, 129, 256, 1000):
        assert H.byte_diff(run((xd[:M],), (wd,), out_dtype=torch.bfloat16), Y[:M]) == 0, M
    gemm = GpuGemm(out_dtype=torch.bfloat16)
    Wn = (normal_bf16(SEED_W, (256, 128)),)
    cells = [H.ab_cell(gemm, H.rows_bf16(256), Wn, M, r) for M in (1, 8, 32) for r in (0, M // 2, M - 1)]
    H.report("bf16 -> bf16 out X[M,256].W[256,128]", cells, K=256, N=128, dtype="bf16")
    assert not [c for c in cells if c["ab"] or c["canon"]]


def test_mxfp8_bf16_output_ab_cells():
    gemm = GpuGemm(out_dtype=torch.bfloat16)
    K, N = 512, 128
    W = (normal_e4m3(SEED_W, (K, N)), e8m0_scales(SEED_W + SCALE_SEED_OFFSET, (K // 32, N), "var"))
    make = H.rows_mx(K, "var")
    cells = [H.ab_cell(gemm, make, W, M, r) for M in (1, 16, 64) for r in (0, M // 2, M - 1)]
    H.report("MXFP8 -> bf16 out", cells, K=K, N=N, dtype="e4m3")
    assert not [c for c in cells if c["ab"] or c["canon"]]


# ------------------------------------------------------------------------- int8
I8_SHAPES = [(1, 16, 16), (33, 272, 160), (130, 256, 1024), (300, 64, 4096), (129, 400, 528)]


@pytest.mark.parametrize("M,N,K", I8_SHAPES)
def test_i8_exact(M, N, K):
    X, W = int_i8(71, (M, K)), int_i8(72, (K, N))
    y = run((dev_i8(X),), (dev_i8(W),))
    assert y.dtype == torch.int32
    assert np.array_equal(y.cpu().numpy().astype(np.int64), oracle.gemm_i8(X, W))


def test_i8_extremes():
    """-128 * -128 summed over K = 4096 (2^26 per element) and mixed 127 / -128."""
    M, N, K = 64, 128, 4096
    X = np.full((M, K), -128, np.int8)
    W = np.full((K, N), -128, np.int8)
    W[:, 1::2] = 127
    y = run((dev_i8(X),), (dev_i8(W),)).cpu().numpy()
    assert (y[:, 0::2] == 4096 * 16384).all() and (y[:, 1::2] == -4096 * 128 * 127).all()


def test_i8_invariance():
    gemm = GpuGemm()
    W = (int_i8(SEED_W, (256, 128)),)
    make = H.rows_i8(256)
    cells = [H.ab_cell(gemm, make, W, M, r) for M in (1, 4, 16, 32) for r in (0, M // 2, M - 1)]
    H.report("int8 X[M,256].W[256,128]", cells, K=256, N=128, dtype="i8")
    assert not [c for c in cells if c["ab"] or c["canon"]]
    xd = dev_i8(int_i8(SEED_X, (1024, 1024)))
    wd = dev_i8(int_i8(SEED_W, (1024, 512)))
    Y = run((xd,), (wd,))
    for M in (1, 7, 64, 65, 129, 256, 1000):
        assert H.byte_diff(run((xd[:M],), (wd,)), Y[:M]) == 0, M
