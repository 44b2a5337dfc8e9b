"""Batch-invariant RMSNorm on the GPU through the C ABI: parity with the oracle's
binary64 RMSNorm within the derived fp32 (+ bf16 output) bound, and byte-level
batch invariance with the GEMM harness's cells (gamma in the weight's place)."""
import numpy as np
import pytest
import torch

import harness as H
import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import SEED_W, SEED_X, normal_bf16
from gpu_util import DEV, dev_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def rms(x, g, eps=1e-6, out=None):
    y = bg.rmsnorm(x, g, eps, out=out)
    torch.cuda.synchronize()
    return y


def to_f64(y):
    if y.dtype == torch.float32:
        return y.cpu().numpy().astype(np.float64)
    return y.cpu().view(torch.bfloat16).float().numpy().astype(np.float64)


def _check(y, ref, D, bf16_out):
    tol = oracle.rmsnorm_tol(D, bf16_out)
    err = np.abs(to_f64(y) - ref)
    bound = tol * np.abs(ref) + 1e-30
    assert (err <= bound).all(), float((err / (np.abs(ref) + 1e-30)).max())


SHAPES = [(1, 8), (7, 4096), (300, 1024), (64, 8192), (5, 8200), (33, 520), (2, 65536)]


@pytest.mark.parametrize("M,D", SHAPES)
def test_rmsnorm_bf16_parity(M, D):
    X, G = normal_bf16(91, (M, D)), normal_bf16(92, (D,))
    y = rms(dev_bf16(X), dev_bf16(G))
    _check(y, oracle.rmsnorm(X, G, 1e-6), D, True)


@pytest.mark.parametrize("M,D", SHAPES)
def test_rmsnorm_f32_parity(M, D):
    rng = np.random.default_rng(93)
    X = (rng.standard_normal((M, D)) * 3).astype(np.float32)
    G = rng.standard_normal(D).astype(np.float32)
    y = rms(torch.from_numpy(X).to(DEV), torch.from_numpy(G).to(DEV), 0.25)
    _check(y, oracle.rmsnorm(X, G, 0.25), D, False)


def test_rmsnorm_in_place_nan_and_zero_rows():
    X, G = normal_bf16(94, (16, 1024)), normal_bf16(95, (1024,))
    X[4, 17] = 0x7FC0      # NaN in row 4 only
    X[9, :] = 0            # zero row: 0 / sqrt(eps) = 0
    xd, gd = dev_bf16(X), dev_bf16(G)
    y = rms(xd, gd)
    yh = to_f64(y)
    assert np.isnan(yh[4]).all() and (yh[9] == 0).all()
    others = [i for i in range(16) if i != 4]
    assert H.byte_diff(y[others], rms(xd[others].contiguous(), gd)) == 0
    inplace = xd.clone()
    rms(inplace, gd, out=inplace)
    assert H.byte_diff(inplace, y) == 0


def test_rmsnorm_bad_args_and_m_zero():
    xd, gd = dev_bf16(normal_bf16(96, (4, 64))), dev_bf16(normal_bf16(97, (64,)))
    y = torch.empty_like(xd)
    assert bg.bigemm_rmsnorm(bg.BIGEMM_BF16, 0, 64, 0, 64, 0, 0, 64, 1e-6) == bg.BIGEMM_OK
    assert bg.bigemm_rmsnorm(bg.BIGEMM_BF16, 4, 60, xd.data_ptr(), 64, gd.data_ptr(), y.data_ptr(), 64, 1e-6,
                             check=False) == bg.BIGEMM_ERR_ARG


class _Norm:
    def __call__(self, batch, weights):
        return rms(dev_bf16(batch[0]), dev_bf16(weights[0]))


def test_rmsnorm_ab_position_and_msweep():
    norm = _Norm()
    G = (normal_bf16(SEED_W, (4096,)),)
    make = H.rows_bf16(4096)
    cells = [H.ab_cell(norm, make, G, M, r) for M in (1, 4, 8, 16, 32, 300) for r in (0, M // 2, M - 1)]
    H.report("RMSNorm D=4096", cells, K=4096, N=4096, dtype="bf16")
    assert not [c for c in cells if c["ab"] or c["canon"]]
    for M in (17, 129):
        assert all(v == 0 for v in H.position_cell(norm, make, G, M).values()), M
    xd = dev_bf16(normal_bf16(SEED_X, (2048, 4096)))
    gd = dev_bf16(G[0])
    Y = rms(xd, gd)
    for M in (1, 7, 64, 65, 256, 1000, 2047):
        assert H.byte_diff(rms(xd[:M], gd), Y[:M]) == 0, M
