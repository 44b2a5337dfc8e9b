"""CPU GEMMs for the harness self-test (test infrastructure).

Positive controls (batch invariant by construction) and negative controls
that change a row's reduction with the batch, which the harness must catch —
the vLLM mHC PR insists on controls that actually fail, at realistic
magnitudes (section "Tests"):

* NC1 — K split into max(1, n_cu // ceil(M/64)) contiguous chunks merged in
  order: the batch-dependent split count of the PR's compute_num_split
  (section "What"); caught by the M sweep across the 64-row boundaries.
* NC2 — per-tensor amax scaling of X over the whole batch: a row's rounding
  then depends on the other rows' contents (the content-dependent class the
  CANN issue's VAR-scale trigger belongs to); caught by the A/B cell.
* NC3 — the K split depends on which 16-row tile holds the row (stream-K-like
  per-tile splits, the blog's batch-invariant matmul section); caught by the
  position cell.

All arithmetic here is float32 with an explicit k-ascending accumulation
order, so the only batch dependence is the one each control plants.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _decode(batch, weights):
    """Decoded float64 operands (torch CPU conversions); scales applied if present."""
    x = batch[0]
    w = weights[0]
    if x.dtype == np.uint16:
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double().numpy()
        wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).double().numpy()
        return xd, wd
    xd = torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e4m3fn).float().double().numpy()
    wd = torch.from_numpy(np.ascontiguousarray(w)).view(torch.float8_e4m3fn).float().double().numpy()
    xd = np.ldexp(xd, np.repeat(batch[1].astype(np.int64) - 127, 32, axis=1))
    wd = np.ldexp(wd, np.repeat(weights[1].astype(np.int64) - 127, 32, axis=0))
    return xd, wd


def _ordered_f32(x32, w32, k_lo, k_hi):
    """sum_{k=k_lo}^{k_hi-1} x[:, k] w[k, :] in float32, k ascending."""
    acc = np.zeros((x32.shape[0], w32.shape[1]), dtype=np.float32)
    for k in range(k_lo, k_hi):
        acc += x32[:, k:k + 1] * w32[k:k + 1, :]
    return acc


# ------------------------------------------------------------------ positive
def gemm_oracle(batch, weights):
    """The fp64 oracle rounded once to float32 — batch invariant by construction."""
    if batch[0].dtype == np.uint16:
        y = oracle.gemm_bf16(batch[0], weights[0], want_s=False)
    else:
        y = oracle.gemm_mxfp8(batch[0], weights[0], batch[1], weights[1], want_s=False)
    return y.astype(np.float32)


def gemm_ordered_f32(batch, weights):
    """One float32 accumulation order for every row — batch invariant by construction."""
    xd, wd = _decode(batch, weights)
    x32, w32 = xd.astype(np.float32), wd.astype(np.float32)
    return _ordered_f32(x32, w32, 0, x32.shape[1])


# ------------------------------------------------------------------ negative
def _split_sum(x32, w32, splits):
    K = x32.shape[1]
    splits = max(1, min(splits, K))
    bounds = [K * s // splits for s in range(splits + 1)]
    out = np.zeros((x32.shape[0], w32.shape[1]), dtype=np.float32)
    for s in range(splits):
        out += _ordered_f32(x32, w32, bounds[s], bounds[s + 1])
    return out


def gemm_nc1_msplit(batch, weights, n_cu: int = 256):
    xd, wd = _decode(batch, weights)
    M = xd.shape[0]
    splits = max(1, n_cu // -(-M // 64))
    return _split_sum(xd.astype(np.float32), wd.astype(np.float32), splits)


def gemm_nc2_amax(batch, weights):
    xd, wd = _decode(batch, weights)
    x32 = xd.astype(np.float32)
    s = np.float32(np.abs(x32).max())
    if s == 0:
        s = np.float32(1.0)
    xs = x32 / s
    return _ordered_f32(xs, wd.astype(np.float32), 0, x32.shape[1]) * s


def gemm_nc3_position(batch, weights, tile_rows: int = 16):
    xd, wd = _decode(batch, weights)
    x32, w32 = xd.astype(np.float32), wd.astype(np.float32)
    out = np.zeros((x32.shape[0], w32.shape[1]), dtype=np.float32)
    for t0 in range(0, x32.shape[0], tile_rows):
        splits = 1 + (t0 // tile_rows) % 3
        out[t0:t0 + tile_rows] = _split_sum(x32[t0:t0 + tile_rows], w32, splits)
    return out
