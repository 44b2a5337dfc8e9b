"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph), as a
serving loop would capture a decode step: the GEMM in both W layouts, the
opt-in split-K with a preallocated workspace, the RMSNorm, the KV-cache write
and the paged attention. The library allocates nothing and issues no memset,
so the captured graph is its kernels alone. The graph is replayed several
times with the program's own eager work (fills of the outputs, other library
calls) and synchronisations between replays, and every replay's outputs must
equal the eager results bit for bit."""
import numpy as np
import pytest
import torch

import invariant_gemm_deterministic_amd as bg
from bigemm_inputs import block_table, kv_bf16, normal_bf16
from gpu_util import DEV, dev_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_graph_replays_match_eager():
    M, N, K = 257, 1000, 1096
    x = dev_bf16(normal_bf16(1, (M, K)))
    w = dev_bf16(normal_bf16(2, (K, N), 0.05))
    w_nk = w.t().contiguous()
    k_chunk = 256
    ws = torch.empty(bg.bigemm_workspace_size(bg._handle("bf16", 0, bg.BIGEMM_F32, k_chunk), M, N, K),
                     dtype=torch.uint8, device=DEV)
    xr = dev_bf16(normal_bf16(3, (64, 4096)))
    gamma = dev_bf16(normal_bf16(4, (4096,)))

    # decode: one token per sequence at its last position, the token's K/V written first
    lens, hkv, h, d, bs = [300, 1, 513, 64], 2, 8, 128, 32
    kh, vh = kv_bf16(5, lens, hkv, d)
    bt, nblocks = block_table(6, lens, bs, 2)
    kc = torch.zeros((nblocks, hkv, bs, d), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = torch.zeros_like(kc)
    seqs = np.arange(len(lens), dtype=np.int32)
    last = np.array(lens, dtype=np.int32) - 1
    bt_d, seqs_d, last_d = _i32(bt), _i32(seqs), _i32(last)
    earlier = np.concatenate([np.full(L - 1, s) for s, L in enumerate(lens)]).astype(np.int32)
    earlier_pos = np.concatenate([np.arange(L - 1) for L in lens]).astype(np.int32)
    bg.kv_cache_write(dev_bf16(kh[earlier, earlier_pos]).view(torch.bfloat16),
                      dev_bf16(vh[earlier, earlier_pos]).view(torch.bfloat16), kc, vc, bt_d, _i32(earlier),
                      _i32(earlier_pos))
    k_new = dev_bf16(kh[seqs, last]).view(torch.bfloat16)
    v_new = dev_bf16(vh[seqs, last]).view(torch.bfloat16)
    q = dev_bf16(normal_bf16(7, (len(lens), h, d))).view(torch.bfloat16)
    max_context = bt.shape[1] * bs
    aws = torch.empty(bg.bigemm_attn_workspace_size(bg._kv_layout(kc, bt_d), len(lens), h, max_context),
                      dtype=torch.uint8, device=DEV)

    def outputs():
        return {"y": torch.empty((M, N), device=DEV), "y_nk": torch.empty((M, N), device=DEV),
                "y_split": torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
                "norm": torch.empty_like(xr), "attn": torch.empty((len(lens), h, d), device=DEV)}

    def step(o):
        bg.mm(x, w, out=o["y"])
        bg.mm(x, w_nk.t(), out=o["y_nk"])
        bg.mm(x, w, out=o["y_split"], k_chunk=k_chunk, workspace=ws)
        bg.rmsnorm(xr, gamma, 1e-6, out=o["norm"])
        bg.kv_cache_write(k_new, v_new, kc, vc, bt_d, seqs_d, last_d)
        bg.paged_attention(q, kc, vc, bt_d, seqs_d, last_d, max_context=max_context, out=o["attn"], workspace=aws)

    eager = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(eager)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}

    captured = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(captured)
    torch.cuda.synchronize()

    other = torch.empty((M, N), device=DEV)
    for replay in range(4):
        for v in captured.values():
            v.fill_(-3.0)                       # eager fill kernels between replays
        bg.mm(x[: 7 + replay], w, out=other[: 7 + replay])   # an eager library call of another shape
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(_bits(captured[k]), _bits(ref[k])), (replay, k)
    assert torch.equal(_bits(other[:10]), _bits(ref["y"][:10]))   # rows of the eager call equal the batch's
    assert torch.isfinite(ref["attn"]).all()
