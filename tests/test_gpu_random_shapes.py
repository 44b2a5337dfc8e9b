"""Seeded random shapes across every input family (bf16, fp16, MXFP8 with K-varying scales, int8), with
random row padding of every operand: each row's bytes are the same computed alone, inside a random
sub-batch and inside the full batch, and sampled rows agree with the oracle (exactly for int8)."""
import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import e8m0_scales, int_i8, normal_bf16, normal_e4m3, normal_f16
from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu

SHAPES_PER_FAMILY = 60


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class _Padded:
    """A device copy of a 2-D array whose rows carry 0-2 extra 16-byte units of padding; indexing
    gathers rows (keeping the padded row length) and returns the [rows, cols] view."""

    def __init__(self, a, rng, dtype):
        rows, cols = a.shape
        per = 16 // a.dtype.itemsize
        ld = -(-cols // per) * per + per * int(rng.integers(0, 3))
        buf = np.zeros((rows, ld), dtype=a.dtype)
        buf[:, :cols] = a
        raw = {1: np.uint8, 2: np.int16}[a.dtype.itemsize]
        self.t = torch.from_numpy(buf.view(raw)).to(DEV).view(dtype)
        self.cols = cols

    def __getitem__(self, rows):
        return self.t[rows][:, :self.cols]


def _shape(fam, rng):
    M = int(rng.integers(1, 700))
    if fam in ("bf16", "f16"):
        return M, int(rng.integers(1, 600)), int(rng.integers(1, 3000))
    if fam == "mx":
        return M, 16 * int(rng.integers(1, 40)), 32 * int(rng.integers(1, 96))
    return M, 16 * int(rng.integers(1, 40)), 16 * int(rng.integers(1, 190))


@pytest.mark.parametrize("fam", ["bf16", "f16", "mx", "i8"])
def test_random_shapes_invariance_and_parity(fam):
    rng = np.random.default_rng({"bf16": 101, "f16": 102, "mx": 103, "i8": 104}[fam])
    for _ in range(SHAPES_PER_FAMILY):
        M, N, K = _shape(fam, rng)
        seed = int(rng.integers(0, 1 << 30))
        XS = WS = None
        if fam == "bf16":
            X, W = normal_bf16(seed, (M, K)), normal_bf16(seed + 1, (K, N), 0.05)
            xd, wd = _Padded(X, rng, torch.bfloat16), _Padded(W, rng, torch.bfloat16)
        elif fam == "f16":
            X, W = normal_f16(seed, (M, K)), normal_f16(seed + 1, (K, N), 0.05)
            xd, wd = _Padded(X, rng, torch.float16), _Padded(W, rng, torch.float16)
        elif fam == "mx":
            X, W = normal_e4m3(seed, (M, K)), normal_e4m3(seed + 1, (K, N))
            XS, WS = e8m0_scales(seed + 2, (M, K // 32), "var"), e8m0_scales(seed + 3, (K // 32, N), "var")
            xd, wd = _Padded(X, rng, torch.uint8), _Padded(W, rng, torch.uint8)
            xsd, wsd = _Padded(XS, rng, torch.uint8), _Padded(WS, rng, torch.uint8)
        else:
            X, W = int_i8(seed, (M, K)), int_i8(seed + 1, (K, N))
            xd, wd = _Padded(X, rng, torch.int8), _Padded(W, rng, torch.int8)
        w = wd[slice(None)]

        def mm(rows):
            if fam == "mx":
                return bg.mm(xd[rows], w, xsd[rows], wsd[slice(None)])
            return bg.mm(xd[rows], w)

        sub = np.sort(rng.choice(M, size=max(1, M // 3), replace=False))
        r = int(rng.integers(0, M))
        full, part, alone = mm(slice(None)), mm(torch.from_numpy(sub).to(DEV)), mm(slice(r, r + 1))
        torch.cuda.synchronize()
        bits = lambda t: t.cpu().view(torch.int32)
        fb = bits(full)
        case = f"{fam} M={M} N={N} K={K} seed={seed}"
        assert torch.equal(bits(part), fb[torch.from_numpy(sub)]), case
        assert torch.equal(bits(alone), fb[r:r + 1]), case
        rows = np.unique(np.array([0, r, M - 1]))
        y = full.cpu().numpy()[rows]
        if fam == "i8":
            assert np.array_equal(y.astype(np.int64), oracle.gemm_i8(X[rows], W)), case
            continue
        if fam == "bf16":
            Y, S = oracle.gemm_bf16(X[rows], W)
        elif fam == "f16":
            Y, S = oracle.gemm_f16(X[rows], W)
        else:
            Y, S = oracle.gemm_mxfp8(X[rows], W, XS[rows], WS)
        assert oracle.max_normalized_error(y, Y, S) <= oracle.PARITY_TOL, case
