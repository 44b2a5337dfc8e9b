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
    x = batch[0]
    if x.dtype == np.uint16:
        return (dev_bf16(x),)
    return (dev_u8(x), dev_u8(batch[1]))


def run(xd, wd, out=None):
    """Y = X W on the GPU (torch device tensors in; float32 device tensor out), synchronised."""
    if len(xd) == 1:
        y = bg.mm(xd[0], wd[0], out=out)
    else:
        y = bg.mm(xd[0], wd[0], xd[1], wd[1], out=out)
    torch.cuda.synchronize()
    return y


class GpuGemm:
    """Harness adapter: numpy batch and weights in, device float32 result out.
    Weights are uploaded once per weights tuple."""

    def __init__(self):
        self._w = {}

    def __call__(self, batch, weights):
        key = id(weights)
        if key not in self._w:
            self._w[key] = (weights, to_dev(weights))
        return run(to_dev(batch), self._w[key][1])


def rows_alone(xd, wd, rows):
    """Each requested row computed on its own (M = 1)."""
    return [run(tuple(a[r:r + 1] for a in xd), wd)[0] for r in rows]
