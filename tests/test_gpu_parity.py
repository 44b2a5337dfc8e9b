"""GPU results against the CPU oracle, through the C ABI.

Gate (written here, derived from the blog's sequential-sum bound): the maximum
over elements of |y_gpu - y_oracle| / sum_k |x_ik w_kj| must not exceed 2e-3;
integer-valued operands (every partial sum exact in fp32) must match the
oracle bit for bit. Full comparisons at sizes the oracle finishes quickly
(several tiles plus ragged tails) and at every workload size whose fp64 product
costs at most about 100 GFLOP; 256 sampled rows (all columns) above that.
"""
import numpy as np
import pytest
import torch

import oracle
from bigemm_inputs import (SEED_W, SEED_X, normal_bf16, int_bf16, linspace_bf16, normal_e4m3, int_e4m3,
                           e8m0_scales, e8m0_kvar_scales)
from gpu_util import DEV, dev_bf16, dev_u8, require_gpu, run
import invariant_gemm_deterministic_amd as bg

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _parity_bf16(X, W, rows=None):
    y = run((dev_bf16(X),), (dev_bf16(W),)).cpu().numpy()
    if rows is None:
        Y, S = oracle.gemm_bf16(X, W)
        return oracle.max_normalized_error(y, Y, S)
    Y, S = oracle.gemm_bf16(X[rows], W)
    return oracle.max_normalized_error(y[rows], Y, S)


BF16_SHAPES = [  # (M, N, K): one tile, ragged tails in M, N and K, multi-tile
    (1, 128, 256), (4, 128, 256), (8, 128, 256), (16, 128, 256), (32, 128, 256),
    (1, 8, 8), (3, 24, 40), (127, 136, 72), (129, 264, 520), (300, 1000, 1096),
    (513, 512, 4096), (257, 4096, 512),
]


@pytest.mark.parametrize("M,N,K", BF16_SHAPES)
def test_bf16_parity(M, N, K):
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N))
    assert _parity_bf16(X, W) <= TOL


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (5, 40, 24), (130, 264, 200), (257, 128, 4096), (64, 1024, 2048)])
def test_bf16_integer_exact(M, N, K):
    X = int_bf16(5, (M, K))
    W = int_bf16(6, (K, N))
    y = run((dev_bf16(X),), (dev_bf16(W),)).cpu().numpy()
    Y = oracle.gemm_bf16(X, W, want_s=False)
    assert np.array_equal(y.astype(np.float64), Y)


def test_bf16_leading_dimensions():
    """Padded rows (ld > width) read and write only the logical matrix."""
    M, N, K = 70, 136, 96
    X = normal_bf16(1, (M, K + 24))
    W = normal_bf16(2, (K, N + 8))
    xd = dev_bf16(X)[:, :K]
    wd = dev_bf16(W)[:, :N]
    out = torch.full((M, N + 4), -7.0, device=DEV)
    y = bg.mm(xd, wd, out=out[:, :N])
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(np.ascontiguousarray(X[:, :K]), np.ascontiguousarray(W[:, :N]))
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL
    assert torch.all(out[:, N:] == -7.0)


def test_bf16_largest_leading_dimensions():
    """Leading dimensions at the documented limit (128 * ld * element size just below 2^31): the
    kernel's 32-bit tile offsets reach 2.1e9 bytes and stay exact; one element more is rejected."""
    M, N, K = 200, 136, 64
    ldx = ldw = (1 << 23) - 8          # bf16: 128 * ld * 2 = 2^31 - 2048
    ldy = (1 << 22) - 4                # fp32: 128 * ld * 4 = 2^31 - 2048
    X = normal_bf16(31, (M, K))
    W = normal_bf16(32, (K, N))
    xb = torch.empty(M * ldx, dtype=torch.int16, device=DEV)
    wb = torch.empty(K * ldw, dtype=torch.int16, device=DEV)
    yb = torch.full((M * ldy,), -7.0, device=DEV)
    xd = xb.as_strided((M, K), (ldx, 1))
    wd = wb.as_strided((K, N), (ldw, 1))
    yd = yb.as_strided((M, N), (ldy, 1))
    xd.copy_(torch.from_numpy(X.view(np.int16)))
    wd.copy_(torch.from_numpy(W.view(np.int16)))
    bg.mm(xd, wd, out=yd)
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(yd.cpu().numpy(), Y, S) <= TOL
    assert torch.all(yb.as_strided((M, 8), (ldy, 1), N) == -7.0)   # past each row's N columns
    h = bg._handle("bf16", 0)
    args = dict(x=xd.data_ptr(), w=wd.data_ptr(), y=yd.data_ptr())
    for lx, lw, ly in ((ldx + 8, ldw, ldy), (ldx, ldw + 8, ldy), (ldx, ldw, ldy + 4)):
        assert bg.bigemm_run(h, M, N, K, args["x"], lx, args["w"], lw, args["y"], ly,
                             check=False) == bg.BIGEMM_ERR_ARG
    del xb, wb, yb
    torch.cuda.empty_cache()


def test_bf16_m_zero_is_noop_and_bad_args_rejected():
    xd = dev_bf16(normal_bf16(1, (4, 64)))
    wd = dev_bf16(normal_bf16(2, (64, 32)))
    h = bg._handle("bf16", 0)
    y = torch.full((4, 32), 3.0, device=DEV)
    assert bg.bigemm_run(h, 0, 32, 64, xd.data_ptr(), 64, wd.data_ptr(), 32, y.data_ptr(), 32) == bg.BIGEMM_OK
    # misaligned X, X rows not 16-byte aligned (ldx = 60), scales on a bf16 handle: rejected, nothing written
    assert bg.bigemm_run(h, 4, 32, 64, xd.data_ptr() + 2, 64, wd.data_ptr(), 32, y.data_ptr(), 32,
                         check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run(h, 4, 32, 60, xd.data_ptr(), 60, wd.data_ptr(), 32, y.data_ptr(), 32,
                         check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run(h, 4, 32, 64, xd.data_ptr(), 64, wd.data_ptr(), 32, y.data_ptr(), 32,
                         xd.data_ptr(), 2, wd.data_ptr(), 32, check=False) == bg.BIGEMM_ERR_ARG
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
    assert bg.bigemm_get_config(h) == (128, 128, 64)


def test_bf16_nan_stays_in_its_row():
    """A NaN in one input row poisons that row only (rows never mix)."""
    M, N, K = 40, 256, 512
    X = normal_bf16(3, (M, K))
    W = normal_bf16(4, (K, N))
    y0 = run((dev_bf16(X),), (dev_bf16(W),))
    X2 = X.copy()
    X2[7, 100] = 0x7FC0  # bf16 quiet NaN
    y1 = run((dev_bf16(X2),), (dev_bf16(W),))
    assert torch.isnan(y1[7]).all()
    others = [i for i in range(M) if i != 7]
    assert torch.equal(y1[others].view(torch.int32), y0[others].view(torch.int32))


def test_bf16_tall_batch():
    """Many tiles along M (the grid's largest dimension here)."""
    M, N, K = 1 << 17, 16, 64
    X = normal_bf16(9, (M, K))
    W = normal_bf16(10, (K, N))
    rows = np.array([0, 1, 127, 128, 65535, M // 2, M - 129, M - 1])
    assert _parity_bf16(X, W, rows) <= TOL


def test_linspace_workload_parity():
    """The blog's linspace operands (rounded to bf16), a[2048,4096] . b[4096,4096]: every
    element against the oracle (68.7 GFLOP of fp64 work)."""
    B, D = 2048, 4096
    a = linspace_bf16(-1000.0, 1000.0, B * D, (B, D))
    b = linspace_bf16(-1000.0, 1000.0, D * D, (D, D))
    assert _parity_bf16(a, b) <= TOL


def _sample_rows(M, n, seed):
    """n distinct rows of M: 0, 1, mid, last, the rows around every 1024-row boundary, and
    seeded random rows for the rest."""
    fixed = {0, 1, M // 2, M - 1} | {r for t in range(1024, M, 1024) for r in (t - 1, t)}
    rest = np.setdiff1d(np.arange(M), np.fromiter(fixed, int))
    pick = np.random.default_rng(seed).choice(rest, n - len(fixed), replace=False)
    return np.sort(np.concatenate([np.fromiter(fixed, int), pick]))


@pytest.mark.parametrize("N", [4096, 14336])
def test_projection_full_size_sampled(N):
    """X[4096,4096] ~ N(0,1), W[4096,N] ~ N(0,0.02): 256 sampled rows (0, mid, last, the
    rows at each 1024-row boundary and seeded random rows), every column of each."""
    M = K = 4096
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N), 0.02)
    rows = _sample_rows(M, 256, 0)
    assert len(rows) == 256 and {0, M // 2, M - 1} <= set(rows.tolist())
    assert _parity_bf16(X, W, rows) <= TOL


def test_long_k_full_size():
    """[1024,16384] . [16384,1024], N(0,1): every element (34.4 GFLOP of fp64 work)."""
    M, K, N = 1024, 16384, 1024
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N))
    assert _parity_bf16(X, W) <= TOL


# ---------------------------------------------------------------------- MXFP8
def _mx_inputs(M, N, K, xk, wk, seed=0, integer=False):
    if integer:
        X, W = int_e4m3(40 + seed, (M, K)), int_e4m3(41 + seed, (K, N))
    else:
        X, W = normal_e4m3(40 + seed, (M, K)), normal_e4m3(41 + seed, (K, N))
    if xk == "kvar":
        XS = e8m0_kvar_scales(42 + seed, K // 32, M, k_axis=1)
    else:
        XS = e8m0_scales(42 + seed, (M, K // 32), xk)
    if wk == "kvar":
        WS = e8m0_kvar_scales(43 + seed, K // 32, N, k_axis=0)
    else:
        WS = e8m0_scales(43 + seed, (K // 32, N), wk)
    return X, W, XS, WS


def _run_mx(X, W, XS, WS):
    return run((dev_u8(X), dev_u8(XS)), (dev_u8(W), dev_u8(WS))).cpu().numpy()


MX_SHAPES = [(1, 64, 128), (4, 128, 256), (64, 512, 2048), (33, 256, 160), (130, 272, 1024), (300, 64, 96)]
COMBOS = [("id", "id"), ("id", "var"), ("var", "id"), ("var", "var"), ("kvar", "kvar")]


@pytest.mark.parametrize("M,N,K", MX_SHAPES)
@pytest.mark.parametrize("xk,wk", COMBOS)
def test_mxfp8_parity(M, N, K, xk, wk):
    X, W, XS, WS = _mx_inputs(M, N, K, xk, wk)
    y = _run_mx(X, W, XS, WS)
    Y, S = oracle.gemm_mxfp8(X, W, XS, WS)
    assert oracle.max_normalized_error(y, Y, S) <= TOL


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (65, 256, 160), (200, 512, 2048)])
def test_mxfp8_integer_exact_id_scales(M, N, K):
    X, W, XS, WS = _mx_inputs(M, N, K, "id", "id", integer=True)
    y = _run_mx(X, W, XS, WS)
    assert np.array_equal(y.astype(np.float64), oracle.gemm_mxfp8(X, W, XS, WS, want_s=False))


def test_mxfp8_integer_exact_small_var_scales():
    """VAR scales with every partial sum exact in fp32: K * 64 * 2^8 < 2^24."""
    M, N, K = 40, 96, 256
    X, W, XS, WS = _mx_inputs(M, N, K, "var", "var", integer=True)
    XS = np.clip(XS, 125, 129).astype(np.uint8)
    WS = np.clip(WS, 125, 129).astype(np.uint8)
    y = _run_mx(X, W, XS, WS)
    assert np.array_equal(y.astype(np.float64), oracle.gemm_mxfp8(X, W, XS, WS, want_s=False))


def test_mxfp8_scale_shift_bit_identical():
    """2^s moved from X's K block b to W's block b: bit-identical GPU output."""
    M, N, K = 48, 128, 512
    X, W, XS, WS = _mx_inputs(M, N, K, "var", "var")
    y0 = _run_mx(X, W, XS, WS)
    XS2, WS2 = XS.copy(), WS.copy()
    XS2[:, 3] += 2
    WS2[3, :] -= 2
    y1 = _run_mx(X, W, XS2, WS2)
    assert y0.tobytes() == y1.tobytes()


@pytest.mark.parametrize("K", [1024, 2048])
def test_mxfp8_scale_load_paths_bit_identical(K):
    """Scales reach the kernel either staged through LDS in groups of four K
    blocks (X and W scale rows 16-byte aligned, K a multiple of 512) or one byte
    at a time (any other layout). Both paths must give the same bytes: compare
    packed scales with the same values in padded rows and at an odd base address,
    for X scales and for W scales."""
    M, N = 200, 256
    X, W, XS, WS = _mx_inputs(M, N, K, "var", "var", seed=7)
    y_packed = _run_mx(X, W, XS, WS)
    nsb = K // 32
    wide = torch.zeros((M, nsb + 5), dtype=torch.uint8, device=DEV)
    wide[:, :nsb] = dev_u8(XS)     # rows nsb + 5 bytes apart: not a multiple of 16
    y_padded = run((dev_u8(X), wide[:, :nsb]), (dev_u8(W), dev_u8(WS))).cpu().numpy()
    wide.zero_()
    wide[:, 1:1 + nsb] = dev_u8(XS)  # base one byte past an aligned allocation
    y_odd = run((dev_u8(X), wide[:, 1:1 + nsb]), (dev_u8(W), dev_u8(WS))).cpu().numpy()
    assert y_packed.tobytes() == y_padded.tobytes()
    assert y_packed.tobytes() == y_odd.tobytes()
    wide_w = torch.zeros((nsb, N + 5), dtype=torch.uint8, device=DEV)
    wide_w[:, :N] = dev_u8(WS)     # W scale rows N + 5 bytes apart
    y_wpad = run((dev_u8(X), dev_u8(XS)), (dev_u8(W), wide_w[:, :N])).cpu().numpy()
    wide_w.zero_()
    wide_w[:, 1:1 + N] = dev_u8(WS)  # W scales one byte past an aligned allocation
    y_wodd = run((dev_u8(X), dev_u8(XS)), (dev_u8(W), wide_w[:, 1:1 + N])).cpu().numpy()
    assert y_packed.tobytes() == y_wpad.tobytes()
    assert y_packed.tobytes() == y_wodd.tobytes()


@pytest.mark.parametrize("K", [160, 1024])
def test_mxfp8_nan_scale_stays_in_its_row(K):
    """A NaN X scale (E8M0 0xFF) in one row poisons that row only."""
    M, N = 48, 128
    X, W, XS, WS = _mx_inputs(M, N, K, "var", "var", seed=3)
    y0 = _run_mx(X, W, XS, WS)
    XS2 = XS.copy()
    XS2[5, :] = 255
    y1 = _run_mx(X, W, XS2, WS)
    others = np.arange(M) != 5
    assert y1[others].tobytes() == y0[others].tobytes()
    assert np.isnan(y1[5]).all()


def test_mxfp8_large_full():
    """MXFP8 X[512,4096] . W[4096,4096] with K-varying scales on both sides: every element."""
    M, N, K = 512, 4096, 4096
    X, W, XS, WS = _mx_inputs(M, N, K, "var", "var")
    y = _run_mx(X, W, XS, WS)
    Y, S = oracle.gemm_mxfp8(X, W, XS, WS)
    assert oracle.max_normalized_error(y, Y, S) <= TOL
