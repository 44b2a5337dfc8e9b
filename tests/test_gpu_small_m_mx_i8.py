"""MXFP8 and int8 products with tiles of at most 64 rows, through the C ABI.

In such a tile each wave of the MXFP8 and int8 kernels (4 waves of 64 x 64 outputs) runs the K loop
for the number of its 32-row fragments and of its X loads that hold a row below M: fragments holding
only rows past M are neither read nor multiplied, and X loads of rows past M are left out (six loops,
chosen per wave; tiles of more than 64 rows run the full loop). Checked here for every count of rows in
a tile from 1 to 130 (and 255):
- MXFP8, both scale-load paths (staged: scale rows 16-byte aligned and K a multiple of 512; byte loads:
  any other layout), W as [K, N] and as [N, K] rows, fp32 and bf16 output: every row's bytes equal the
  same row computed inside a full tile; parity with the oracle on the reference rows; seeded random
  shapes against the oracle and against rows inside a full tile;
- int8, both W layouts: every row equal to numpy's exact int64 product.
With at most 128 tiles and K >= 1985 both kernels pad the grid with prefetch workgroups, which store
nothing: MXFP8 rows from such grids equal the same rows inside an unpadded product, and int8 stays
exact.
"""
import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import e8m0_scales, normal_e4m3
from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def rows_u8(a, width):
    """Device copy of a [R, C] byte array in rows of `width` >= C bytes (zero padding);
    returns the [R, C] view."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    R, C = a.shape
    buf = torch.zeros((R, width), dtype=torch.uint8, device=DEV)
    buf[:, :C] = torch.from_numpy(a).to(DEV)
    return buf[:, :C]


def up16(n):
    return -(-n // 16) * 16


def operands(X, W, XS, WS, path, wt):
    """Device operands. path "staged": scale rows 16-byte aligned (K must be a multiple of 512);
    "byte": scale rows 5 bytes longer than a multiple of 16. wt: W and its scales as the
    transposed views of [N, K] and [N, K/32] arrays."""
    K, N = W.shape
    nsb = K // 32
    sw = (lambda n: up16(n)) if path == "staged" else (lambda n: up16(n) + 5)
    x = rows_u8(X, up16(K))
    xs = rows_u8(XS, sw(nsb))
    if wt:
        w = rows_u8(W.T, up16(K)).t()
        ws = rows_u8(WS.T, sw(nsb)).t()
    else:
        w = rows_u8(W, up16(N))
        ws = rows_u8(WS, sw(N))
    return x, xs, w, ws


def same_bytes(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def mx_inputs(seed, M, N, K):
    X = normal_e4m3(seed, (M, K))
    W = normal_e4m3(seed + 1, (K, N))
    XS = e8m0_scales(seed + 100, (M, K // 32), "var")
    WS = e8m0_scales(seed + 101, (K // 32, N), "var")
    return X, W, XS, WS


@pytest.mark.parametrize("path", ["staged", "byte"])
@pytest.mark.parametrize("wt", [False, True])
def test_mxfp8_every_partial_tile_row_count(path, wt):
    """Every count of rows in a tile, 1 to 130 and 255: each product's rows must equal the same
    rows of one product of 256 rows, whose two tile rows are full (every wave on the full loop)."""
    K, N, BIG = 2048, 304, 256   # N: two full tile columns and a ragged one (MXFP8 needs N % 16 == 0)
    X, W, XS, WS = mx_inputs(120, BIG, N, K)
    x, xs, w, ws = operands(X, W, XS, WS, path, wt)
    ref = bg.mm(x, w, xs, ws)
    torch.cuda.synchronize()
    bad = []
    for m in list(range(1, 131)) + [255]:
        y = bg.mm(x[:m], w, xs[:m], ws)
        torch.cuda.synchronize()
        if not same_bytes(y, ref[:m]):
            bad.append(m)
    assert not bad, f"rows differ from the full-tile product at M = {bad}"
    rows = np.array([0, 1, 7, 8, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, BIG - 1])
    Y, S = oracle.gemm_mxfp8(X[rows], W, XS[rows], WS)
    assert oracle.max_normalized_error(ref.cpu().numpy()[rows], Y, S) <= TOL


@pytest.mark.parametrize("path", ["staged", "byte"])
def test_mxfp8_partial_rows_bf16_out(path):
    """bf16 output at the counts where a wave's loop changes (fragment and X-load boundaries)."""
    K, N, BIG = 1024, 256, 256
    X, W, XS, WS = mx_inputs(130, BIG, N, K)
    x, xs, w, ws = operands(X, W, XS, WS, path, False)
    ref = bg.mm(x, w, xs, ws, out_dtype=torch.bfloat16)
    ref32 = bg.mm(x, w, xs, ws)
    torch.cuda.synchronize()
    assert same_bytes(ref, ref32.to(torch.bfloat16))   # one rounding of the fp32 result
    bad = []
    for m in (1, 2, 8, 9, 16, 17, 24, 25, 32, 33, 40, 41, 48, 49, 56, 57, 64, 65, 96, 97, 128, 129, 160):
        y = bg.mm(x[:m], w, xs[:m], ws, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        if not same_bytes(y, ref[:m]):
            bad.append(m)
    assert not bad, f"rows differ from the full-tile product at M = {bad}"


def test_mxfp8_random_small_m_shapes():
    """16 seeded random shapes with at most 130 rows (K a multiple of 32 up to 4096, N a multiple of 16 up to 992,
    either scale path, either W layout): parity with the oracle, and rows equal to the same rows
    placed first in a product of 256 rows (full tiles)."""
    rng = np.random.default_rng(2027)
    for case in range(16):
        M = int(rng.integers(1, 131))
        N = 16 * int(rng.integers(1, 63))
        path = "staged" if rng.integers(0, 2) else "byte"
        K = 512 * int(rng.integers(1, 9)) if path == "staged" else 32 * int(rng.integers(1, 129))
        wt = bool(rng.integers(0, 2))
        X, W, XS, WS = mx_inputs(3000 + 10 * case, 256, N, K)
        x, xs, w, ws = operands(X, W, XS, WS, path, wt)
        y = bg.mm(x[:M], w, xs[:M], ws)
        big = bg.mm(x, w, xs, ws)
        torch.cuda.synchronize()
        label = f"case {case}: M={M} N={N} K={K} path={path} wt={wt}"
        Y, S = oracle.gemm_mxfp8(X[:M], W, XS[:M], WS)
        assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL, label
        assert same_bytes(y, big[:M]), label


@pytest.mark.parametrize("wt", [False, True])
def test_int8_every_partial_tile_row_count(wt):
    """int8 -> int32: every count of rows in a tile, 1 to 130 and 255, equal to the exact product
    (K * 127^2 < 2^31), W as [K, N] and as [N, K] rows; N with a ragged tile column."""
    K, N, BIG = 2048, 304, 256
    rng = np.random.default_rng(140)
    X = rng.integers(-128, 128, size=(BIG, K)).astype(np.int8)
    W = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    exact = X.astype(np.int64) @ W.astype(np.int64)
    x = rows_u8(X.view(np.uint8), K).view(torch.int8)
    w = (rows_u8(np.ascontiguousarray(W.T).view(np.uint8), K).view(torch.int8).t() if wt
         else rows_u8(W.view(np.uint8), up16(N)).view(torch.int8))
    bad = []
    for m in list(range(1, 131)) + [255]:
        y = bg.mm(x[:m], w)
        torch.cuda.synchronize()
        if not np.array_equal(y.cpu().numpy().astype(np.int64), exact[:m]):
            bad.append(m)
    assert not bad, f"rows differ from the exact product at M = {bad}"


@pytest.mark.parametrize("path", ["staged", "byte"])
@pytest.mark.parametrize("wt", [False, True])
def test_mxfp8_padded_grid_rows_equal_unpadded(path, wt):
    """With at most 128 tiles and K >= 1985 the MXFP8 grid is padded with prefetch workgroups (one
    per CU), which store nothing: rows 1, 37 and 100 of such products (32 tiles) must equal the same
    rows inside a product of 5 x 32 = 160 tiles (a grid that is not padded)."""
    K, N, BIG = 2048, 4096, 640
    X, W, XS, WS = mx_inputs(150, BIG, N, K)
    x, xs, w, ws = operands(X, W, XS, WS, path, wt)
    big = bg.mm(x, w, xs, ws)
    torch.cuda.synchronize()
    for m in (1, 37, 100):
        y = bg.mm(x[:m], w, xs[:m], ws)
        torch.cuda.synchronize()
        assert same_bytes(y, big[:m]), f"M = {m}"
    rows = np.array([0, 36, 99, 639])
    Y, S = oracle.gemm_mxfp8(X[rows], W, XS[rows], WS)
    assert oracle.max_normalized_error(big.cpu().numpy()[rows], Y, S) <= TOL


def test_int8_padded_grid_exact():
    """int8 with a padded grid (32 tiles, K = 4096): exact against numpy's int64 product, rows of M = 1,
    64 and 128."""
    K, N = 4096, 4096
    rng = np.random.default_rng(160)
    X = rng.integers(-128, 128, size=(128, K)).astype(np.int8)
    W = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    exact = X.astype(np.int64) @ W.astype(np.int64)
    x = rows_u8(X.view(np.uint8), K).view(torch.int8)
    w = rows_u8(W.view(np.uint8), N).view(torch.int8)
    for m in (1, 64, 128):
        y = bg.mm(x[:m], w)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.int64), exact[:m]), f"M = {m}"


@pytest.mark.parametrize("path,wt", [("staged", False), ("byte", True)])
def test_mxfp8_long_k_padded_grid(path, wt):
    """64 x 1024 x 16384 (8 tiles, 128 K blocks of 128: the prefetch workgroups walk the whole K with
    the W-scale touches): rows equal to the same rows inside a product of 17 x 8 = 136 tiles (not
    padded), and parity with the oracle on sampled rows."""
    K, N, BIG = 16384, 1024, 2176
    X, W, XS, WS = mx_inputs(170, BIG, N, K)
    x, xs, w, ws = operands(X, W, XS, WS, path, wt)
    big = bg.mm(x, w, xs, ws)
    y = bg.mm(x[:64], w, xs[:64], ws)
    torch.cuda.synchronize()
    assert same_bytes(y, big[:64])
    rows = np.array([0, 31, 63])
    Y, S = oracle.gemm_mxfp8(X[rows], W, XS[rows], WS)
    assert oracle.max_normalized_error(y.cpu().numpy()[rows], Y, S) <= TOL


@pytest.mark.parametrize("wt", [False, True])
def test_int8_long_k_padded_grid_exact(wt):
    """int8 64 x 1024 x 16384 (8 tiles, padded grid): exact against numpy's int64 product (K * 127^2 < 2^31)."""
    K, N = 16384, 1024
    rng = np.random.default_rng(180)
    X = rng.integers(-128, 128, size=(64, K)).astype(np.int8)
    W = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    exact = X.astype(np.int64) @ W.astype(np.int64)
    x = rows_u8(X.view(np.uint8), K).view(torch.int8)
    w = (rows_u8(np.ascontiguousarray(W.T).view(np.uint8), K).view(torch.int8).t() if wt
         else rows_u8(W.view(np.uint8), N).view(torch.int8))
    y = bg.mm(x, w)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.int64), exact)
