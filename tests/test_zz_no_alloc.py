"""bigemm_run_split_k_static (the entry point for callers that cannot allocate: the split-K
chunk sums live in the library's static device buffer) against bigemm_run_ws with a caller
workspace on the same handle, through the C ABI: identical bytes on consecutive calls, the
second one smaller than the first, for both W layouts and both output types; oversize shapes
and handles without split-K are refused before anything is launched."""
import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import normal_bf16
from gpu_util import DEV, dev_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(h, x, w, wt, out_dtype, M, N, K):
    """Y from bigemm_run_ws (torch workspace) and from bigemm_run_split_k_static on handle h."""
    stream = torch.cuda.current_stream().cuda_stream
    wd = w.t() if wt else w                      # logical [K, N]
    ldw = int(w.stride(0))
    y_ws = torch.full((M, N), -3.0, device=DEV).to(out_dtype)
    y_st = torch.full((M, N), -5.0, device=DEV).to(out_dtype)
    need = bg.bigemm_workspace_size(h, M, N, K)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    bg.bigemm_run_ws(h, M, N, K, x.data_ptr(), K, wd.data_ptr(), ldw, y_ws.data_ptr(), N, workspace=ws.data_ptr(),
                     workspace_bytes=need, stream=stream)
    bg.bigemm_run_split_k_static(h, M, N, K, x.data_ptr(), K, wd.data_ptr(), ldw, y_st.data_ptr(), N, stream=stream)
    torch.cuda.synchronize()
    return y_ws, y_st


@pytest.mark.parametrize("wt", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_static_scratch_matches_workspace_on_consecutive_calls(wt, out):
    yt = bg.BIGEMM_F32 if out == "f32" else bg.BIGEMM_BF16
    odt = torch.float32 if out == "f32" else torch.bfloat16
    h = (bg.bigemm_create_split_k_wt if wt else bg.bigemm_create_split_k)(bg.BIGEMM_BF16, bg.BIGEMM_BF16, yt, 512)
    try:
        # first call: 8 chunks of 300 x 4096 (39 MB of chunk sums); second call smaller: 3 chunks of 70 x 136
        for M, N, K, seed in ((300, 4096, 4096, 11), (70, 136, 1096, 12)):
            X = normal_bf16(seed, (M, K))
            W = normal_bf16(seed + 1, (N, K) if wt else (K, N))
            y_ws, y_st = _both(h, dev_bf16(X), dev_bf16(W), wt, odt, M, N, K)
            assert torch.equal(y_ws.view(torch.int16 if out == "bf16" else torch.int32),
                               y_st.view(torch.int16 if out == "bf16" else torch.int32)), (M, N, K)
            if out == "f32":   # and both within the parity bound of the oracle
                Wk = np.ascontiguousarray(W.T) if wt else W
                rows = np.array([0, M // 2, M - 1])
                Y, S = oracle.gemm_bf16(X[rows], Wk)
                assert oracle.max_normalized_error(y_st.cpu().numpy()[rows], Y, S) <= oracle.PARITY_TOL
    finally:
        bg.bigemm_destroy(h)


def test_static_scratch_limits():
    h = bg.bigemm_create_split_k(bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F32, 512)
    try:
        K, N = 4096, 4096
        M = bg.STATIC_SCRATCH_BYTES // (8 * N * 4)        # exactly fills the buffer: 512 rows
        x = dev_bf16(normal_bf16(13, (M + 1, K)))
        w = dev_bf16(normal_bf16(14, (K, N)))
        y = torch.full((M + 1, N), 7.0, device=DEV)
        st = bg.bigemm_run_split_k_static(h, M + 1, N, K, x.data_ptr(), K, w.data_ptr(), N, y.data_ptr(), N,
                                          check=False)
        torch.cuda.synchronize()
        assert st == bg.BIGEMM_ERR_SCRATCH and torch.all(y == 7.0)
        assert "static scratch" in bg.bigemm_status_str(st)
        y_ws, y_st = _both(h, x[:M], w, False, torch.float32, M, N, K)
        assert torch.equal(y_ws.view(torch.int32), y_st.view(torch.int32))
        # one chunk (K <= k_chunk): no scratch needed, the unsplit kernel's bytes
        y1 = torch.empty((M, N), device=DEV)
        bg.bigemm_run_split_k_static(h, M, N, 512, x.data_ptr(), K, w.data_ptr(), N, y1.data_ptr(), N)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), bg.mm(x[:M, :512], w[:512]).view(torch.int32))
    finally:
        bg.bigemm_destroy(h)
    plain = bg.bigemm_create(bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F32)
    try:
        assert bg.bigemm_run_split_k_static(plain, 4, 8, 8, 16, 8, 16, 8, 16, 8, check=False) == bg.BIGEMM_ERR_ARG
    finally:
        bg.bigemm_destroy(plain)
