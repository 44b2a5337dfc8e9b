"""Small-M products through the C ABI: grids padded with prefetch workgroups, and tiles whose
waves skip the fragments and X loads that hold only rows past M.

The bf16 / fp16 kernel pads its grid to one workgroup per CU when the 128 x 128 tiles fill at
most half of the CUs (at most 128 tiles on the 256-CU MI355X) and K spans at least 32 K blocks
(K >= 1985). The extra workgroups of each XCD share out the K blocks of the distinct X and W
panels of the XCD's tiles, touch their lines ahead and store nothing. In a tile with rows past M, each wave runs the K loop for the number of its
fragments and X loads that hold rows below M. Checked here, over tile counts from 2 to 128 (XCDs
with no tile, XCDs holding one tile more than others), K from 32 blocks to 256, K and N not
multiples of 8, every count of rows in a tile from 1 to 130, both W layouts, fp16 inputs and
bf16 output:
- parity with the oracle, and integer-exact inputs bit for bit;
- every row's bytes equal to the same row inside a product of more than 128 tiles (a grid
  that is not padded, every wave on the full-tile loop), with the rows placed first and last.
"""
import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import SEED_W, SEED_X, int_bf16, normal_bf16, normal_f16
from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL

# (M, N, K): tiles
CASES = [
    (1, 4096, 4096),     # 32 tiles, 4 per XCD
    (37, 1000, 2048),    # 8 tiles, one per XCD; 32 K blocks, the fewest that pad
    (300, 1100, 2112),   # 27 tiles: three XCDs hold one tile more
    (129, 128, 8192),    # 2 tiles: six XCDs hold none
    (512, 4096, 4096),   # 128 tiles, the largest padded grid
    (64, 1024, 16384),   # 8 tiles, 256 K blocks
    (100, 520, 4099),    # 5 tiles, K not a multiple of 8
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def dev_rows(a, dtype=torch.int16):
    """Device copy of a [R, C] array of 16-bit values in rows of roundup(C, 8) elements
    (zero padding); returns the [R, C] view."""
    a = np.ascontiguousarray(a)
    R, C = a.shape
    ld = -(-C // 8) * 8
    buf = torch.zeros((R, ld), dtype=torch.int16, device=DEV)
    buf[:, :C] = torch.from_numpy(a.view(np.int16)).to(DEV)
    return buf.view(dtype)[:, :C]


def w_operand(W, wt, dtype=torch.int16):
    """W [K, N] as the kernel operand: [K, N] rows, or the transposed view of [N, K] rows."""
    return dev_rows(np.ascontiguousarray(W.T), dtype).t() if wt else dev_rows(W, dtype)


def unpadded_rows(x, w, out_dtype=None):
    """The rows of x computed inside a product of more than 128 tiles: x placed first and
    last among other rows (seeded normal values). Returns the two [M, N] results."""
    M, K = x.shape
    N = w.shape[1]
    tiles_n = -(-N // 128)
    big = max(128 * (128 // tiles_n + 1), -(-2 * M // 128) * 128)   # tiles_m * tiles_n > 128
    g = torch.Generator(device=DEV)
    g.manual_seed(9001)
    fill = torch.randn((big, K), generator=g, device=DEV)
    fill = fill.to(torch.bfloat16).view(torch.int16) if x.dtype == torch.int16 else fill.to(x.dtype)
    buf = torch.zeros((big, x.stride(0)), dtype=x.dtype, device=DEV)
    buf[:, :K] = fill
    buf[:M, :K] = x
    buf[big - M:, :K] = x
    y = bg.mm(buf[:, :K], w, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y[:M], y[big - M:]


def same_bytes(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("M,N,K", CASES)
def test_prefetch_grid_parity_and_rows(M, N, K):
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N), 0.02)
    x, w = dev_rows(X), w_operand(W, False)
    y = bg.mm(x, w)
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL
    first, last = unpadded_rows(x, w)
    assert same_bytes(y, first) and same_bytes(y, last)


@pytest.mark.parametrize("M,N,K", [(300, 1100, 2112), (100, 520, 4099)])
def test_prefetch_grid_integer_exact(M, N, K):
    X, W = int_bf16(80, (M, K)), int_bf16(81, (K, N))
    y = bg.mm(dev_rows(X), w_operand(W, False))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.gemm_bf16(X, W, want_s=False))


@pytest.mark.parametrize("M,N,K", [(37, 1000, 2048), (100, 520, 4099)])
def test_prefetch_grid_w_transposed(M, N, K):
    """W given as [N, K] rows: the same bytes as the [K, N] layout, and as the rows inside
    an unpadded grid."""
    X = normal_bf16(82, (M, K))
    W = normal_bf16(83, (K, N), 0.02)
    x = dev_rows(X)
    y = bg.mm(x, w_operand(W, False))
    yt = bg.mm(x, w_operand(W, True))
    torch.cuda.synchronize()
    assert same_bytes(y, yt)
    first, last = unpadded_rows(x, w_operand(W, True))
    assert same_bytes(yt, first) and same_bytes(yt, last)


@pytest.mark.parametrize("M,N,K", [(129, 128, 8192), (100, 520, 4099)])
def test_prefetch_grid_f16_and_bf16_out(M, N, K):
    """fp16 inputs and bf16 output: parity, and rows as in an unpadded grid."""
    Xh = normal_f16(84, (M, K))
    Wh = normal_f16(85, (K, N), 0.02)
    xh, wh = dev_rows(Xh, torch.float16), w_operand(Wh, False, torch.float16)
    yh = bg.mm(xh, wh)
    torch.cuda.synchronize()
    Y, S = oracle.gemm_f16(Xh, Wh)
    assert oracle.max_normalized_error(yh.cpu().numpy(), Y, S) <= TOL
    first, last = unpadded_rows(xh, wh)
    assert same_bytes(yh, first) and same_bytes(yh, last)

    X = normal_bf16(86, (M, K))
    W = normal_bf16(87, (K, N), 0.02)
    x, w = dev_rows(X), w_operand(W, False)
    y16 = bg.mm(x, w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y16.float().cpu().numpy(), Y, S) <= oracle.PARITY_TOL_BF16_OUT
    first, last = unpadded_rows(x, w, out_dtype=torch.bfloat16)
    assert same_bytes(y16, first) and same_bytes(y16, last)


def test_every_partial_tile_row_count():
    """Every count of rows in a tile, 1 to 130 (and 255, 256): the waves choose their K loop from
    how many of their fragments and X loads hold rows below M (six combinations occur). Each
    product's rows must equal the same rows of one product of more than 128 tiles (not padded,
    every wave on the full-tile loop). K = 2048 pads the small grids with prefetch workgroups."""
    K, N, BIG = 2048, 2048, 1152   # 16 tile columns; 9 x 16 = 144 tiles for the reference
    X = normal_bf16(90, (BIG, K))
    W = normal_bf16(91, (K, N), 0.02)
    x, w = dev_rows(X), w_operand(W, False)
    ref = bg.mm(x, w)
    torch.cuda.synchronize()
    bad = []
    for m in list(range(1, 131)) + [255, 256]:
        y = bg.mm(x[:m], w)
        torch.cuda.synchronize()
        if not same_bytes(y, ref[:m]):
            bad.append(m)
    assert not bad, f"rows differ from the unpadded product at M = {bad}"
    # the reference itself against the oracle on a sample of rows (every partial count shares them)
    rows = np.array([0, 1, 31, 32, 33, 63, 64, 65, 96, 97, 127, 128, 129, BIG - 1])
    Y, S = oracle.gemm_bf16(X[rows], W)
    assert oracle.max_normalized_error(ref.cpu().numpy()[rows], Y, S) <= TOL


@pytest.mark.parametrize("wt,f16", [(True, False), (False, True)])
def test_partial_tile_row_counts_other_kernels(wt, f16):
    """The same for W given as [N, K] rows and for fp16 inputs, at the counts where a wave's
    choice changes (fragment and X-load boundaries)."""
    K, N, BIG = 2048, 2048, 1152
    dt = torch.float16 if f16 else torch.int16
    X = normal_f16(92, (BIG, K)) if f16 else normal_bf16(92, (BIG, K))
    W = normal_f16(93, (K, N), 0.02) if f16 else normal_bf16(93, (K, N), 0.02)
    x, w = dev_rows(X, dt), w_operand(W, wt, dt)
    ref = bg.mm(x, w)
    torch.cuda.synchronize()
    bad = []
    for m in (1, 2, 8, 9, 16, 17, 24, 25, 32, 33, 40, 41, 56, 57, 64, 65, 72, 73, 96, 97, 104, 105, 120, 121, 127, 128):
        y = bg.mm(x[:m], w)
        torch.cuda.synchronize()
        if not same_bytes(y, ref[:m]):
            bad.append(m)
    assert not bad, f"rows differ from the unpadded product at M = {bad}"


def test_random_small_m_shapes():
    """24 seeded random shapes with few tiles and K of at least 32 blocks (padded grids, every
    combination of row counts, K and N not multiples of 8, both W layouts, bf16 and fp16 inputs,
    fp32 and bf16 output): parity with the oracle, and rows equal to the same rows placed first
    and last in a product of more than 128 tiles."""
    rng = np.random.default_rng(2026)
    for case in range(24):
        M = int(rng.integers(1, 301))
        N = int(rng.integers(1, 3001))
        K = int(rng.integers(1985, 6001))
        wt = bool(rng.integers(0, 2))
        f16 = bool(rng.integers(0, 2))
        out_bf16 = bool(rng.integers(0, 2))
        dt = torch.float16 if f16 else torch.int16
        gen = normal_f16 if f16 else normal_bf16
        X = gen(1000 + case, (M, K))
        W = gen(2000 + case, (K, N), 0.02)
        x, w = dev_rows(X, dt), w_operand(W, wt, dt)
        odt = torch.bfloat16 if out_bf16 else None
        y = bg.mm(x, w, out_dtype=odt)
        torch.cuda.synchronize()
        Y, S = (oracle.gemm_f16 if f16 else oracle.gemm_bf16)(X, W)
        tol = oracle.PARITY_TOL_BF16_OUT if out_bf16 else TOL
        label = f"case {case}: M={M} N={N} K={K} wt={wt} f16={f16} bf16_out={out_bf16}"
        assert oracle.max_normalized_error(y.float().cpu().numpy(), Y, S) <= tol, label
        first, last = unpadded_rows(x, w, out_dtype=odt)
        assert same_bytes(y, first) and same_bytes(y, last), label
