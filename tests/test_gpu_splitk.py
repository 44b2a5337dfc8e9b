"""Opt-in split-K (a K chunk fixed per handle, chunk sums added in ascending order)
on the GPU through the C ABI: parity with the oracle, byte-level batch invariance,
equality with the unsplit kernel for a single chunk, and workspace checks."""
import numpy as np
import pytest
import torch

import harness as H
import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import SEED_W, SEED_X, normal_bf16, normal_f16
from gpu_util import DEV, dev_bf16, require_gpu, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def split(xd, wd, k_chunk, out_dtype=None):
    y = bg.mm(xd, wd, out_dtype=out_dtype, k_chunk=k_chunk)
    torch.cuda.synchronize()
    return y


def dev_f16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(DEV)


@pytest.mark.parametrize("M,N,K,kc", [(1, 128, 4096, 512), (33, 264, 4096, 1024), (130, 256, 1000, 256),
                                      (257, 128, 2048, 128)])
def test_split_k_parity(M, N, K, kc):
    X, W = normal_bf16(81, (M, K)), normal_bf16(82, (K, N))
    y = split(dev_bf16(X), dev_bf16(W), kc).cpu().numpy()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y, Y, S) <= oracle.PARITY_TOL


def test_split_k_f16_parity():
    X, W = normal_f16(83, (70, 512)), normal_f16(84, (512, 136))
    y = split(dev_f16(X), dev_f16(W), 128).cpu().numpy()
    Y, S = oracle.gemm_f16(X, W)
    assert oracle.max_normalized_error(y, Y, S) <= oracle.PARITY_TOL


@pytest.mark.parametrize("K,kc", [(512, 512), (200, 1024)])
def test_single_chunk_is_the_unsplit_kernel(K, kc):
    """K <= k_chunk: one chunk, so the bytes are those of the unsplit handle."""
    xd, wd = dev_bf16(normal_bf16(85, (150, K))), dev_bf16(normal_bf16(86, (K, 256)))
    assert H.byte_diff(split(xd, wd, kc), run((xd,), (wd,))) == 0


def test_split_k_msweep_and_alone():
    K, N, kc = 4096, 512, 512
    xd = dev_bf16(normal_bf16(SEED_X, (1024, K)))
    wd = dev_bf16(normal_bf16(SEED_W, (K, N), 0.02))
    Y = split(xd, wd, kc)
    for M in (1, 7, 8, 63, 64, 65, 128, 129, 193, 256, 1000):
        assert H.byte_diff(split(xd[:M], wd, kc), Y[:M]) == 0, M
    for r in (0, 511, 1023):
        assert H.byte_diff(split(xd[r:r + 1], wd, kc)[0], Y[r]) == 0, r


class _SplitGemm:
    def __init__(self, kc):
        self.kc = kc

    def __call__(self, batch, weights):
        return split(dev_bf16(batch[0]), dev_bf16(weights[0]), self.kc)


def test_split_k_ab_and_position_cells():
    gemm = _SplitGemm(256)
    W = (normal_bf16(SEED_W, (1024, 128)),)
    make = H.rows_bf16(1024)
    cells = [H.ab_cell(gemm, make, W, M, r) for M in (1, 4, 16, 32) for r in (0, M // 2, M - 1)]
    H.report("split-K bf16 X[M,1024].W[1024,128]", cells, K=1024, N=128, dtype="bf16")
    assert not [c for c in cells if c["ab"] or c["canon"]]
    for M in (17, 129):
        assert all(v == 0 for v in H.position_cell(gemm, make, W, M).values()), M


def test_split_k_bf16_output_is_the_rounded_f32_output():
    from test_gpu_dtypes import bf16_bits, rne_bf16_bits
    xd, wd = dev_bf16(normal_bf16(87, (100, 2048))), dev_bf16(normal_bf16(88, (2048, 264)))
    y32 = split(xd, wd, 512).cpu().numpy()
    ybf = split(xd, wd, 512, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(ybf), rne_bf16_bits(y32))


def test_split_k_long_k_workload():
    """[1024,16384] . [16384,1024]: chunks of 2048 (8 per tile, 512 workgroups instead of
    64); sampled parity and invariance for M in {1, 64, 1024}."""
    M, K, N = 1024, 16384, 1024
    X, W = normal_bf16(SEED_X, (M, K)), normal_bf16(SEED_W, (K, N))
    xd, wd = dev_bf16(X), dev_bf16(W)
    Y = split(xd, wd, 2048)
    rows = np.array([0, 511, 1023])
    Yo, So = oracle.gemm_bf16(X[rows], W)
    assert oracle.max_normalized_error(Y[rows].cpu().numpy(), Yo, So) <= oracle.PARITY_TOL
    for m in (1, 64):
        assert H.byte_diff(split(xd[:m], wd, 2048), Y[:m]) == 0, m


def test_split_k_workspace_rules():
    """A short or misaligned workspace is rejected before anything is launched, and a
    split-K handle refuses bigemm_run (it needs a workspace)."""
    M, N, K, kc = 8, 128, 1024, 256
    xd, wd = dev_bf16(normal_bf16(89, (M, K))), dev_bf16(normal_bf16(90, (K, N)))
    y = torch.full((M, N), 7.0, device=DEV)
    h = bg._handle("bf16", 0, bg.BIGEMM_F32, kc)
    need = bg.bigemm_workspace_size(h, M, N, K)
    assert need == 4 * M * N * 4
    assert bg.bigemm_workspace_size(h, M, N, kc) == 0            # one chunk: no workspace
    ws = torch.empty(need + 64, dtype=torch.uint8, device=DEV)
    args = (h, M, N, K, xd.data_ptr(), K, wd.data_ptr(), N, y.data_ptr(), N, 0, 0, 0, 0)
    assert bg.bigemm_run_ws(*args, ws.data_ptr(), need - 4, 0, check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run_ws(*args, ws.data_ptr() + 4, need, 0, check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run_ws(*args, 0, need, 0, check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run(*args, 0, check=False) == bg.BIGEMM_ERR_ARG
    torch.cuda.synchronize()
    assert (y == 7.0).all()                                      # nothing was written
    assert bg.bigemm_run_ws(*args, ws.data_ptr(), need, 0, check=False) == bg.BIGEMM_OK
    torch.cuda.synchronize()
    assert not (y == 7.0).all()


@pytest.mark.parametrize("N", [128, 130])
def test_split_k_merge_adds_chunk_sums_in_ascending_order(N):
    """Each chunk sum is the unsplit kernel's product over that K slice (the same MFMA chain from zero),
    and the merge adds the chunk sums in ascending order in fp32: rebuilt on the CPU from unsplit calls
    on the K slices, the split-K output matches bit for bit. 20 chunks cover the merge's look-ahead
    groups of 8 and a partial group; N = 130 takes the one-output-per-thread merge (W rows padded to
    keep them 16-byte aligned)."""
    M, K, kc = 37, 2560, 128
    X = normal_bf16(91, (M, K))
    Wp = np.zeros((K, 136), dtype=X.dtype)
    Wp[:, :N] = normal_bf16(92, (K, N))
    xd, wpd = dev_bf16(X), dev_bf16(Wp)
    wd = wpd[:, :N]
    y = split(xd, wd, kc).cpu().numpy()
    acc = None
    for c in range(K // kc):
        yc = run((xd[:, c * kc:(c + 1) * kc],), (wpd[c * kc:(c + 1) * kc, :N],)).cpu().numpy().astype(np.float32)
        acc = yc if acc is None else (acc + yc).astype(np.float32)
    assert y.dtype == np.float32 and acc.shape == y.shape
    assert np.array_equal(y.view(np.int32), acc.view(np.int32))
