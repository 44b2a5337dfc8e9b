"""bf16 / fp16 inputs whose K or N is not a multiple of 8, through the C ABI.

Rows must still start 16-byte aligned, so the operands sit in padded rows (leading
dimension rounded up to 8 elements). The padding is filled with NaN (X) and infinity (W)
so that any use of it shows: the last 16-byte piece of a row is read whole, X values past
K are zeroed before the multiply, W rows past K are never read and W columns past N only
reach output columns that are not stored. Checked here: parity with the oracle, the same
bytes as the problem zero-padded to a multiple of 8, both W layouts, bf16 output, split-K,
and the A/B, position and M-sweep cells of the harness at K = 4099, N = 129."""
import numpy as np
import pytest
import torch

import harness as H
import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import SEED_W, SEED_X, int_bf16, normal_bf16, normal_f16
from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL
NAN16, INF16 = 0x7FC0, 0x7F80


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def padded(a, fill, dtype=torch.int16):
    """Device copy of a [R, C] array of 16-bit patterns in rows of roundup(C, 8) elements,
    the padding set to the bit pattern `fill`; returns the [R, C] view."""
    a = np.ascontiguousarray(a)
    R, C = a.shape
    ld = -(-C // 8) * 8
    buf = torch.full((R, ld), fill, dtype=torch.int16, device=DEV)
    buf[:, :C] = torch.from_numpy(a.view(np.int16)).to(DEV)
    return buf.view(dtype)[:, :C]


def gemm_padded(X, W, out_dtype=None, k_chunk=None, f16=False, wt=False):
    dt = torch.float16 if f16 else torch.int16
    xd = padded(X, NAN16 if not f16 else 0x7E00, dt)
    if wt:  # W given as [N, K] rows, padded past K
        wd = padded(np.ascontiguousarray(W.T), INF16 if not f16 else 0x7C00, dt).t()
    else:
        wd = padded(W, INF16 if not f16 else 0x7C00, dt)
    y = bg.mm(xd, wd, out_dtype=out_dtype, k_chunk=k_chunk)
    torch.cuda.synchronize()
    return y


SHAPES = [(5, 1, 1), (33, 129, 7), (3, 129, 1), (64, 8, 7), (130, 129, 4099), (257, 1, 4099),
          (200, 264, 4100), (129, 131, 515)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_tail_parity(M, N, K):
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N))
    y = gemm_padded(X, W).cpu().numpy()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y, Y, S) <= TOL


@pytest.mark.parametrize("M,N,K", [(33, 129, 7), (130, 131, 4099)])
def test_tail_integer_exact(M, N, K):
    X, W = int_bf16(70, (M, K)), int_bf16(71, (K, N))
    y = gemm_padded(X, W).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), oracle.gemm_bf16(X, W, want_s=False))


@pytest.mark.parametrize("M,N,K", [(33, 129, 7), (130, 129, 4099), (7, 1, 1)])
def test_tail_equals_zero_padding(M, N, K):
    """The same bytes as the zero-padded problem (K and N rounded up to 8, zeros in the
    padding), which runs the multiple-of-8 kernel: every output element accumulates the
    same products in the same order."""
    X = normal_bf16(72, (M, K))
    W = normal_bf16(73, (K, N))
    Kp, Np = -(-K // 8) * 8, -(-N // 8) * 8
    Xz = np.zeros((M, Kp), np.uint16)
    Xz[:, :K] = X
    Wz = np.zeros((Kp, Np), np.uint16)
    Wz[:K, :N] = W
    y = gemm_padded(X, W)
    yz = bg.mm(torch.from_numpy(Xz.view(np.int16)).to(DEV), torch.from_numpy(Wz.view(np.int16)).to(DEV))
    torch.cuda.synchronize()
    assert H.byte_diff(y, yz[:, :N].contiguous()) == 0
    yb = gemm_padded(X, W, out_dtype=torch.bfloat16)
    ybz = bg.mm(torch.from_numpy(Xz.view(np.int16)).to(DEV), torch.from_numpy(Wz.view(np.int16)).to(DEV),
                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert H.byte_diff(yb, ybz[:, :N].contiguous()) == 0


@pytest.mark.parametrize("M,N,K", [(33, 129, 7), (130, 129, 4099)])
def test_tail_w_transposed_same_bytes(M, N, K):
    """W given as [N, K] rows whose padding past K is infinity: the bytes of the [K, N] call."""
    X = normal_bf16(74, (M, K))
    W = normal_bf16(75, (K, N))
    assert H.byte_diff(gemm_padded(X, W, wt=True), gemm_padded(X, W)) == 0


def test_tail_fp16_parity():
    M, N, K = 70, 129, 1003
    X = normal_f16(76, (M, K))
    W = normal_f16(77, (K, N))
    y = gemm_padded(X, W, f16=True).cpu().numpy()
    Y, S = oracle.gemm_f16(X, W)
    assert oracle.max_normalized_error(y, Y, S) <= TOL


@pytest.mark.parametrize("N", [129, 132])
def test_tail_split_k(N):
    """Split-K with K = 4099 (the last chunk holds the tail) and N = 129 (the merge then adds
    one output per thread) or 132: parity, and a row alone equals its row in the batch."""
    M, K = 70, 4099
    X = normal_bf16(78, (M, K))
    W = normal_bf16(79, (K, N))
    y = gemm_padded(X, W, k_chunk=512)
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL
    for r in (0, 35, 69):
        assert H.byte_diff(gemm_padded(X[r:r + 1], W, k_chunk=512)[0], y[r]) == 0, r


class _Padded:
    def __call__(self, batch, weights):
        return gemm_padded(batch[0], weights[0])


def test_tail_invariance_cells():
    """The harness's cells at K = 4099, N = 129: A/B cells with target rows 0, mid and last,
    position cells, and an M sweep across tile boundaries."""
    K, N = 4099, 129
    g = _Padded()
    W = (normal_bf16(SEED_W, (K, N), 0.02),)
    make = H.rows_bf16(K)
    cells = [H.ab_cell(g, make, W, M, r) for M in (1, 4, 33, 130) for r in (0, M // 2, M - 1)]
    H.report("bf16 tails K=4099 N=129", cells, K=K, N=N, dtype="bf16")
    assert not [c for c in cells if c["ab"] or c["canon"]], cells
    for M in (17, 129):
        assert all(v == 0 for v in H.position_cell(g, make, W, M).values()), M
    sweep = H.msweep_cell(g, (normal_bf16(SEED_X, (300, K)),), W, (1, 7, 128, 129, 257))
    assert all(v["rows"] == 0 and v["alone"] == 0 for v in sweep.values()), sweep


def test_tail_random_shapes():
    """30 seeded random shapes with any K in [1, 1100] and N in [1, 640] (rows padded to
    a multiple of 8 elements plus a random extra 0, 8 or 24, the padding NaN / infinity):
    oracle parity of the fp32 output, the W^T call's bytes equal to the [K, N] call's,
    and the bf16 output equal to the fp32 output rounded once."""
    from test_gpu_dtypes import rne_bf16_bits
    rng = np.random.default_rng(2024)
    for case in range(30):
        M, N, K = int(rng.integers(1, 300)), int(rng.integers(1, 640)), int(rng.integers(1, 1100))
        extra = int(rng.choice([0, 8, 24]))
        X = normal_bf16(500 + case, (M, K))
        W = normal_bf16(600 + case, (K, N))
        Xp = np.full((M, -(-K // 8) * 8 + extra), NAN16, np.uint16)
        Xp[:, :K] = X
        Wp = np.full((K, -(-N // 8) * 8 + extra), INF16, np.uint16)
        Wp[:, :N] = W
        WTp = np.full((N, -(-K // 8) * 8 + extra), INF16, np.uint16)
        WTp[:, :K] = W.T
        xd = torch.from_numpy(Xp.view(np.int16)).to(DEV)[:, :K]
        wd = torch.from_numpy(Wp.view(np.int16)).to(DEV)[:, :N]
        wtd = torch.from_numpy(WTp.view(np.int16)).to(DEV)[:, :K].t()
        y = bg.mm(xd, wd)
        yt = bg.mm(xd, wtd) if N > 1 else y   # one output column: no separate [N, K] layout
        yb = bg.mm(xd, wd, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        Y, S = oracle.gemm_bf16(X, W)
        yh = y.cpu().numpy()
        assert oracle.max_normalized_error(yh, Y, S) <= TOL, (case, M, N, K)
        assert H.byte_diff(y, yt) == 0, (case, M, N, K)
        ybh = yb.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ybh, rne_bf16_bits(np.ascontiguousarray(yh))), (case, M, N, K)
