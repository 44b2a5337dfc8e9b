"""Batch-invariance harness (test infrastructure).

Implements the cell types used to check that an output row's bytes depend only
on that input row and W:

* A/B cell — the CANN ops-transformer issue's Variant A/B contract (section
  "test methodology"): the target row i holds the same content C in both
  variants, every other row comes from seed A or seed B, and the assertion is
  byte(y_A[i]) == byte(y_B[i]); the per-cell metric is the byte-diff count
  (section "ATK integration": > 0 fails). Also compared: the row computed on
  its own (M = 1), the canonical bytes of C.
* position cell — C placed at rows 0, mid = floor(M/2) and last = M-1 of one
  batch; every copy must equal the canonical bytes (the blog's point that
  stream-K even breaks batch-position invariance, section on batch-invariant
  matmul).
* M-sweep cell — prefixes X[:M] of one batch across tile and wave boundaries
  (the vLLM mHC PR's bitwise sweep over batch sizes, section "Tests"); every
  row must equal the same row computed in the largest batch.
* repeat cell — identical calls give identical bytes (the blog's 1000-run
  torch.mm check, introduction).

A "batch" is a tuple of arrays with the batch on axis 0 (X, or X and its
scales); ``gemm(batch, weights) -> float32 [M, N]`` is any implementation.
"""
from __future__ import annotations

import numpy as np

from bigemm_inputs import (SEED_A, SEED_B, SEED_C, SCALE_SEED_OFFSET, normal_bf16, normal_e4m3, normal_f16, int_i8,
                           e8m0_scales, e8m0_kvar_scales, row_positions)


def byte_diff(a, b) -> int:
    """Number of differing bytes between two arrays (numpy, or torch tensors on one
    device) of the same shape and dtype."""
    if type(a).__module__.startswith("torch"):
        import torch
        assert a.shape == b.shape and a.dtype == b.dtype, (a.shape, b.shape)
        ua = a.contiguous().view(-1).view(torch.uint8)
        ub = b.contiguous().view(-1).view(torch.uint8)
        return int((ua != ub).sum().item())
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, (a.shape, b.shape, a.dtype, b.dtype)
    return int(np.count_nonzero(a.view(np.uint8) != b.view(np.uint8)))


# ----------------------------------------------------------------- row makers
def rows_bf16(K: int, sigma: float = 1.0):
    def make(seed: int, n: int):
        return (normal_bf16(seed, (n, K), sigma),)
    return make


def rows_f16(K: int, sigma: float = 1.0):
    """fp16 rows (numpy float16, so the GPU adapter can tell them from bf16 bits)."""
    def make(seed: int, n: int):
        return (normal_f16(seed, (n, K), sigma).view(np.float16),)
    return make


def rows_i8(K: int):
    def make(seed: int, n: int):
        return (int_i8(seed, (n, K)),)
    return make


def rows_mx(K: int, kind: str):
    """E4M3 rows from N(0,1) with their X-scale rows; ``kind`` in {"id", "var", "kvar"}."""
    def make(seed: int, n: int):
        x = normal_e4m3(seed, (n, K))
        if kind == "kvar":
            s = e8m0_kvar_scales(seed + SCALE_SEED_OFFSET, K // 32, n, k_axis=1)
        else:
            s = e8m0_scales(seed + SCALE_SEED_OFFSET, (n, K // 32), kind)
        return (x, s)
    return make


def _with_row(batch, i, row):
    out = tuple(a.copy() for a in batch)
    for a, r in zip(out, row):
        a[i] = r[0]
    return out


# ---------------------------------------------------------------------- cells
def sha256_of(arrays) -> str:
    """sha256 over the bytes of a tuple of arrays (the record of which inputs a cell used)."""
    import hashlib
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def ab_cell(gemm, make_rows, weights, M: int, row: int,
            seed_C: int = SEED_C, seed_A: int = SEED_A, seed_B: int = SEED_B):
    C = make_rows(seed_C, 1)
    XA = _with_row(make_rows(seed_A, M), row, C)
    XB = _with_row(make_rows(seed_B, M), row, C)
    yA = gemm(XA, weights)[row]
    yB = gemm(XB, weights)[row]
    y1 = gemm(C, weights)[0]
    return {"M": M, "row": row, "ab": byte_diff(yA, yB), "canon": byte_diff(yA, y1),
            "degenerate": M == 1, "seeds": [seed_C, seed_A, seed_B], "sha256_C": sha256_of(C),
            "sha256_W": sha256_of(weights)}


# Every A/B cell the GPU tests ran, one record each: the issue's per-cell byte-diff
# count (section "ATK integration"), written as JSON lines to $BIGEMM_BI_REPORT at
# the end of the session and summed in the test summary.
REPORT = []


def report(config: str, cells, **fields):
    for c in cells:
        REPORT.append(dict(config=config, **fields, **c))


def position_cell(gemm, make_rows, weights, M: int, seed_C: int = SEED_C, seed_fill: int = SEED_A):
    C = make_rows(seed_C, 1)
    y1 = gemm(C, weights)[0]
    diffs = {}
    fill = make_rows(seed_fill, M)
    for r in row_positions(M):
        y = gemm(_with_row(fill, r, C), weights)[r]
        diffs[r] = byte_diff(y, y1)
    return diffs


def msweep_cell(gemm, batch, weights, Ms):
    """Every row of every prefix batch[:M] must equal that row in the full batch;
    rows 0, mid and last are also compared with the row computed alone."""
    Mmax = batch[0].shape[0]
    Y = gemm(batch, weights)
    out = {}
    for M in Ms:
        assert M <= Mmax
        YM = gemm(tuple(a[:M] for a in batch), weights)
        rows = byte_diff(YM, Y[:M])
        alone = 0
        for r in row_positions(M):
            alone += byte_diff(gemm(tuple(a[r:r + 1] for a in batch), weights)[0], Y[r])
        out[M] = {"rows": rows, "alone": alone}
    return out


def repeat_cell(gemm, batch, weights, n: int = 3) -> int:
    ys = [gemm(batch, weights) for _ in range(n)]
    return sum(byte_diff(ys[0], y) for y in ys[1:])
