"""GPU-side helpers for the parity and invariance tests: device copies of the
seeded inputs and a call of the C ABI through the binding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg

DEV = torch.device("cuda", 0)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    bg.load()  # raises if libbigemm.so is not built: there is no fallback


def dev_bf16(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_dev(batch):
    """numpy operand tuple -> device tensors: uint16 = bf16 bits, float16 = fp16,
    int8 = int8, uint8 = (E4M3 codes, E8M0 scales)."""
    x = batch[0]
    if x.dtype == np.uint16:
        return (dev_bf16(x),)
    if x.dtype == np.float16:
        return (torch.from_numpy(np.ascontiguousarray(x)).to(DEV),)
    if x.dtype == np.int8:
        return (torch.from_numpy(np.ascontiguousarray(x)).to(DEV),)
    return (dev_u8(x), dev_u8(batch[1]))


def run(xd, wd, out=None, out_dtype=None):
    """Y = X W on the GPU (torch device tensors in; device tensor out), synchronised."""
    if len(xd) == 1:
        y = bg.mm(xd[0], wd[0], out=out, out_dtype=out_dtype)
    else:
        y = bg.mm(xd[0], wd[0], xd[1], wd[1], out=out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


class GpuGemm:
    """Harness adapter: numpy batch and weights in, device result out (float32 unless
    ``out_dtype`` says otherwise). Weights are uploaded once per weights tuple."""

    def __init__(self, out_dtype=None):
        self._w = {}
        self.out_dtype = out_dtype

    def __call__(self, batch, weights):
        key = id(weights)
        if key not in self._w:
            self._w[key] = (weights, to_dev(weights))
        return run(to_dev(batch), self._w[key][1], out_dtype=self.out_dtype)


def rows_alone(xd, wd, rows):
    """Each requested row computed on its own (M = 1)."""
    return [run(tuple(a[r:r + 1] for a in xd), wd)[0] for r in rows]
