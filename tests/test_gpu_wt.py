"""W given as its transpose ([N, K] rows, as a linear layer stores its weight).

The W-transposed handle stages W's tile differently but feeds the MFMA chain
the same operands in the same order, so its output must carry exactly the
bytes of the [K, N] handle for the same logical W (compared as raw bits) at
every shape, ragged tails included; one direct oracle comparison per input
type ties it to the gate of the other parity tests as well.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bigemm_inputs import SEED_W, SEED_X, normal_bf16
from gpu_util import DEV, dev_bf16, require_gpu
import invariant_gemm_deterministic_amd as bg

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(y):
    return y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16)


def _both(xd, wd_kn, wd_nk_t, out_dtype):
    """The [K, N] handle and the W-transposed handle on the same logical W."""
    a = bg.mm(xd, wd_kn, out_dtype=out_dtype)
    b = bg.mm(xd, wd_nk_t, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return a, b


SHAPES = [(1, 8, 8), (3, 24, 40), (127, 136, 72), (129, 264, 520), (300, 1000, 1096),
          (513, 512, 4096), (257, 4096, 512), (1024, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wt_bytes_equal_kn_bf16(M, N, K, out_dtype):
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N))
    xd = dev_bf16(X)
    wt = dev_bf16(np.ascontiguousarray(W.T))            # [N, K] rows
    a, b = _both(xd, dev_bf16(W), wt.t(), out_dtype)
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("M,N,K", [(5, 40, 24), (129, 264, 520), (600, 1024, 2048)])
def test_wt_bytes_equal_kn_fp16(M, N, K):
    g = torch.Generator().manual_seed(M * 7 + N)
    X = torch.randn(M, K, generator=g).to(torch.float16)
    W = torch.randn(K, N, generator=g).to(torch.float16)
    xd, wd = X.to(DEV), W.to(DEV)
    wt = W.t().contiguous().to(DEV)
    for od in (torch.float32, torch.bfloat16):
        a, b = _both(xd, wd, wt.t(), od)
        assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("M,N,K", [(127, 136, 72), (300, 1000, 1096)])
def test_wt_oracle_parity(M, N, K):
    X = normal_bf16(SEED_X + 1, (M, K))
    W = normal_bf16(SEED_W + 1, (K, N))
    y = bg.mm(dev_bf16(X), dev_bf16(np.ascontiguousarray(W.T)).t())
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL


def test_wt_padded_rows_and_rows_independent_of_m():
    """Padded [N, K] rows (ldw > K) read only the logical matrix; a row's bytes do not follow M."""
    M, N, K = 300, 264, 520
    X = normal_bf16(3, (M, K))
    WT = normal_bf16(4, (N, K + 40))                     # rows padded by 40 elements
    wt = dev_bf16(WT)[:, :K]                            # stride (K + 40, 1)
    w_kn = dev_bf16(np.ascontiguousarray(WT[:, :K].T))
    xd = dev_bf16(X)
    a, b = _both(xd, w_kn, wt.t(), torch.float32)
    assert torch.equal(_bits(a), _bits(b))
    for i in (0, 131, M - 1):
        one = bg.mm(xd[i:i + 1], wt.t())
        torch.cuda.synchronize()
        assert torch.equal(_bits(one[0]), _bits(b[i]))


def test_wt_largest_leading_dimension():
    """ldw at the documented limit (128 * ldw * 2 just below 2^31) stays exact; one more is rejected."""
    M, N, K = 200, 136, 64
    ldw = (1 << 23) - 8
    X = normal_bf16(5, (M, K))
    W = normal_bf16(6, (K, N))
    big = torch.zeros((N, ldw), dtype=torch.int16, device=DEV)
    big[:, :K] = dev_bf16(np.ascontiguousarray(W.T))
    xd = dev_bf16(X)
    a, b = _both(xd, dev_bf16(W), big[:, :K].t(), torch.float32)
    assert torch.equal(_bits(a), _bits(b))
    y = torch.empty((M, N), device=DEV)
    h = bg._handle("bf16", 0, bg.BIGEMM_F32, 0, True)
    st = bg.bigemm_run(h, M, N, K, xd.data_ptr(), K, big.data_ptr(), ldw + 8, y.data_ptr(), N, check=False)
    assert st == bg.BIGEMM_ERR_ARG
    del big
    torch.cuda.empty_cache()


def test_wt_handle_rejects_kn_leading_dimension_rules():
    """On a W-transposed handle ldw is checked against K: ldw = N < K is refused before any launch."""
    M, N, K = 16, 64, 256
    xd = dev_bf16(normal_bf16(7, (M, K)))
    wt = dev_bf16(normal_bf16(8, (N, K)))
    y = torch.empty((M, N), device=DEV)
    h = bg._handle("bf16", 0, bg.BIGEMM_F32, 0, True)
    st = bg.bigemm_run(h, M, N, K, xd.data_ptr(), K, wt.data_ptr(), N, y.data_ptr(), N, check=False)
    assert st == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run(h, 0, N, K, 0, K, 0, K, 0, N, check=False) == bg.BIGEMM_OK


def test_wt_create_refuses_other_families():
    for t, sb in ((bg.BIGEMM_E4M3, 32), (bg.BIGEMM_I8, 0)):
        h = ctypes.c_void_p()
        d = bg.bigemm_desc(t, t, bg.BIGEMM_I32 if t == bg.BIGEMM_I8 else bg.BIGEMM_F32, sb)
        assert bg.load().bigemm_create_wt(ctypes.byref(d), ctypes.byref(h)) == bg.BIGEMM_ERR_UNSUPPORTED
        assert h.value is None


def test_mm_transposed_w_limits():
    """The binding takes a transposed w only for bf16 / fp16 without split-K, and never a w with no
    contiguous dimension."""
    xd = dev_bf16(normal_bf16(9, (8, 64)))
    wt = dev_bf16(normal_bf16(10, (128, 64)))
    with pytest.raises(ValueError):
        bg.mm(xd, wt.t(), k_chunk=64)
    w_strided = dev_bf16(normal_bf16(11, (64, 256)))[:, ::2]
    with pytest.raises(ValueError):
        bg.mm(xd, w_strided)
    x8 = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    w8 = torch.zeros((128, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        bg.mm(x8, w8.t())
