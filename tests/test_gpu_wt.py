"""W given as its transpose ([N, K] rows, as a linear layer stores its weight;
for MXFP8 with W_scale as [N, K/32]).

The W-transposed handle stages W's tile (and scales) differently but feeds
the MFMA chain the same operands and scales in the same order, so its output
must carry exactly the bytes of the [K, N] handle for the same logical W
(compared as raw bits) at every shape, ragged tails included, for every input
family and both MXFP8 scale-load paths; direct oracle comparisons tie it to
the gate of the other parity tests as well.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bigemm_inputs import SEED_W, SEED_X, e8m0_scales, int_i8, normal_bf16, normal_e4m3
from gpu_util import DEV, dev_bf16, dev_u8, require_gpu
import invariant_gemm_deterministic_amd as bg

pytestmark = pytest.mark.gpu
TOL = oracle.PARITY_TOL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(y):
    return y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16)


def _both(xd, wd_kn, wd_nk_t, out_dtype):
    """The [K, N] handle and the W-transposed handle on the same logical W."""
    a = bg.mm(xd, wd_kn, out_dtype=out_dtype)
    b = bg.mm(xd, wd_nk_t, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return a, b


SHAPES = [(1, 8, 8), (3, 24, 40), (127, 136, 72), (129, 264, 520), (300, 1000, 1096),
          (513, 512, 4096), (257, 4096, 512), (1024, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wt_bytes_equal_kn_bf16(M, N, K, out_dtype):
    X = normal_bf16(SEED_X, (M, K))
    W = normal_bf16(SEED_W, (K, N))
    xd = dev_bf16(X)
    wt = dev_bf16(np.ascontiguousarray(W.T))            # [N, K] rows
    a, b = _both(xd, dev_bf16(W), wt.t(), out_dtype)
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("M,N,K", [(5, 40, 24), (129, 264, 520), (600, 1024, 2048)])
def test_wt_bytes_equal_kn_fp16(M, N, K):
    g = torch.Generator().manual_seed(M * 7 + N)
    X = torch.randn(M, K, generator=g).to(torch.float16)
    W = torch.randn(K, N, generator=g).to(torch.float16)
    xd, wd = X.to(DEV), W.to(DEV)
    wt = W.t().contiguous().to(DEV)
    for od in (torch.float32, torch.bfloat16):
        a, b = _both(xd, wd, wt.t(), od)
        assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("M,N,K", [(127, 136, 72), (300, 1000, 1096)])
def test_wt_oracle_parity(M, N, K):
    X = normal_bf16(SEED_X + 1, (M, K))
    W = normal_bf16(SEED_W + 1, (K, N))
    y = bg.mm(dev_bf16(X), dev_bf16(np.ascontiguousarray(W.T)).t())
    torch.cuda.synchronize()
    Y, S = oracle.gemm_bf16(X, W)
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL


def test_wt_padded_rows_and_rows_independent_of_m():
    """Padded [N, K] rows (ldw > K) read only the logical matrix; a row's bytes do not follow M."""
    M, N, K = 300, 264, 520
    X = normal_bf16(3, (M, K))
    WT = normal_bf16(4, (N, K + 40))                     # rows padded by 40 elements
    wt = dev_bf16(WT)[:, :K]                            # stride (K + 40, 1)
    w_kn = dev_bf16(np.ascontiguousarray(WT[:, :K].T))
    xd = dev_bf16(X)
    a, b = _both(xd, w_kn, wt.t(), torch.float32)
    assert torch.equal(_bits(a), _bits(b))
    for i in (0, 131, M - 1):
        one = bg.mm(xd[i:i + 1], wt.t())
        torch.cuda.synchronize()
        assert torch.equal(_bits(one[0]), _bits(b[i]))


def test_wt_largest_leading_dimension():
    """ldw at the documented limit (128 * ldw * 2 just below 2^31) stays exact; one more is rejected."""
    M, N, K = 200, 136, 64
    ldw = (1 << 23) - 8
    X = normal_bf16(5, (M, K))
    W = normal_bf16(6, (K, N))
    big = torch.zeros((N, ldw), dtype=torch.int16, device=DEV)
    big[:, :K] = dev_bf16(np.ascontiguousarray(W.T))
    xd = dev_bf16(X)
    a, b = _both(xd, dev_bf16(W), big[:, :K].t(), torch.float32)
    assert torch.equal(_bits(a), _bits(b))
    y = torch.empty((M, N), device=DEV)
    h = bg._handle("bf16", 0, bg.BIGEMM_F32, 0, True)
    st = bg.bigemm_run(h, M, N, K, xd.data_ptr(), K, big.data_ptr(), ldw + 8, y.data_ptr(), N, check=False)
    assert st == bg.BIGEMM_ERR_ARG
    del big
    torch.cuda.empty_cache()


def test_wt_handle_rejects_kn_leading_dimension_rules():
    """On a W-transposed handle ldw is checked against K: ldw = N < K is refused before any launch."""
    M, N, K = 16, 64, 256
    xd = dev_bf16(normal_bf16(7, (M, K)))
    wt = dev_bf16(normal_bf16(8, (N, K)))
    y = torch.empty((M, N), device=DEV)
    h = bg._handle("bf16", 0, bg.BIGEMM_F32, 0, True)
    st = bg.bigemm_run(h, M, N, K, xd.data_ptr(), K, wt.data_ptr(), N, y.data_ptr(), N, check=False)
    assert st == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run(h, 0, N, K, 0, K, 0, K, 0, N, check=False) == bg.BIGEMM_OK


def test_wt_create_refuses_descriptors_not_provided():
    for d in (bg.bigemm_desc(bg.BIGEMM_BF16, bg.BIGEMM_F16, bg.BIGEMM_F32, 0),
              bg.bigemm_desc(bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 16),
              bg.bigemm_desc(bg.BIGEMM_I8, bg.BIGEMM_I8, bg.BIGEMM_F32, 0)):
        h = ctypes.c_void_p()
        assert bg.load().bigemm_create_wt(ctypes.byref(d), ctypes.byref(h)) == bg.BIGEMM_ERR_UNSUPPORTED
        assert h.value is None


@pytest.mark.parametrize("M,N,K,k_chunk", [(1, 136, 1000, 256), (5, 264, 520, 512), (129, 4096, 4096, 512),
                                             (300, 1000, 1096, 2048), (64, 1024, 16384, 2048)])
@pytest.mark.parametrize("dtype,out_dtype", [("bf16", torch.float32), ("bf16", torch.bfloat16),
                                             ("f16", torch.float32)])
def test_wt_split_k_bytes_equal_kn(M, N, K, k_chunk, dtype, out_dtype):
    """Split-K with W as [N, K] rows: the bytes of the [K, N] split-K call with the same k_chunk (a
    ragged last chunk, a single chunk, many chunks)."""
    if dtype == "bf16":
        X, W = normal_bf16(SEED_X + 2, (M, K)), normal_bf16(SEED_W + 2, (K, N))
        xd, w_kn, w_nk = dev_bf16(X), dev_bf16(W), dev_bf16(np.ascontiguousarray(W.T))
    else:
        g = torch.Generator().manual_seed(M + K)
        Xf = torch.randn(M, K, generator=g).to(torch.float16)
        Wf = torch.randn(K, N, generator=g).to(torch.float16)
        xd, w_kn, w_nk = Xf.to(DEV), Wf.to(DEV), Wf.t().contiguous().to(DEV)
    a = bg.mm(xd, w_kn, out_dtype=out_dtype, k_chunk=k_chunk)
    b = bg.mm(xd, w_nk.t(), out_dtype=out_dtype, k_chunk=k_chunk)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))
    if K <= k_chunk:   # one chunk: the unsplit kernel's bytes
        c = bg.mm(xd, w_nk.t(), out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(_bits(c), _bits(b))


def test_wt_split_k_create_refuses_other_families():
    for d in (bg.bigemm_desc(bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 32),
              bg.bigemm_desc(bg.BIGEMM_I8, bg.BIGEMM_I8, bg.BIGEMM_I32, 0)):
        h = ctypes.c_void_p()
        assert bg.load().bigemm_create_split_k_wt(ctypes.byref(d), 512, ctypes.byref(h)) == \
            bg.BIGEMM_ERR_UNSUPPORTED
        assert h.value is None
    h = ctypes.c_void_p()
    d = bg.bigemm_desc(bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F32, 0)
    assert bg.load().bigemm_create_split_k_wt(ctypes.byref(d), 100, ctypes.byref(h)) == bg.BIGEMM_ERR_ARG


def test_mm_transposed_w_limits():
    """The binding takes no w with no contiguous dimension, and no MXFP8 w_scale in a layout other
    than w's."""
    xd = dev_bf16(normal_bf16(9, (8, 64)))
    w_strided = dev_bf16(normal_bf16(11, (64, 256)))[:, ::2]
    with pytest.raises(ValueError):
        bg.mm(xd, w_strided)
    M, N, K = 8, 64, 128
    x = dev_u8(normal_e4m3(1, (M, K)))
    xs = dev_u8(e8m0_scales(2, (M, K // 32), "var"))
    w_nk = dev_u8(normal_e4m3(3, (N, K)))
    ws_kn = dev_u8(e8m0_scales(4, (K // 32, N), "var"))
    with pytest.raises(ValueError):
        bg.mm(x, w_nk.t(), xs, ws_kn)          # w as [N, K] rows, w_scale as [K/32, N] rows


def _mx_case(M, N, K, seed=0):
    X, W = normal_e4m3(40 + seed, (M, K)), normal_e4m3(41 + seed, (K, N))
    XS = e8m0_scales(42 + seed, (M, K // 32), "var")
    WS = e8m0_scales(43 + seed, (K // 32, N), "var")
    return X, W, XS, WS


# K = 160 and 96: byte-path scales; K a multiple of 512 with packed scale rows: staged scales
MX_SHAPES = [(1, 64, 128), (33, 256, 160), (300, 64, 96), (130, 272, 1024), (64, 512, 2048),
             (1024, 4096, 4096)]


@pytest.mark.parametrize("M,N,K", MX_SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wt_bytes_equal_kn_mxfp8(M, N, K, out_dtype):
    X, W, XS, WS = _mx_case(M, N, K)
    xd, xs = dev_u8(X), dev_u8(XS)
    a = bg.mm(xd, dev_u8(W), xs, dev_u8(WS), out_dtype=out_dtype)
    b = bg.mm(xd, dev_u8(W.T).t(), xs, dev_u8(WS.T).t(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("K", [1024, 2048])
def test_wt_mxfp8_scale_load_paths(K):
    """W^T scale rows packed (staged through LDS), padded to a length that is not a multiple of 16,
    or one byte past an aligned base (byte path): all give the bytes of the [K, N] call."""
    M, N = 200, 256
    X, W, XS, WS = _mx_case(M, N, K, seed=7)
    xd, xs = dev_u8(X), dev_u8(XS)
    ref = bg.mm(xd, dev_u8(W), xs, dev_u8(WS))
    w_t = dev_u8(W.T).t()
    nsb = K // 32
    wide = torch.zeros((N, nsb + 5), dtype=torch.uint8, device=DEV)
    outs = []
    wide[:, :nsb] = dev_u8(WS.T)
    outs.append(bg.mm(xd, w_t, xs, wide[:, :nsb].t()))
    torch.cuda.synchronize()
    wide.zero_()
    wide[:, 1:1 + nsb] = dev_u8(WS.T)
    outs.append(bg.mm(xd, w_t, xs, wide[:, 1:1 + nsb].t()))
    outs.append(bg.mm(xd, w_t, xs, dev_u8(WS.T).t()))
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(_bits(y), _bits(ref))


@pytest.mark.parametrize("M,N,K", [(33, 256, 160), (130, 272, 1024)])
def test_wt_mxfp8_oracle_parity(M, N, K):
    X, W, XS, WS = _mx_case(M, N, K, seed=3)
    y = bg.mm(dev_u8(X), dev_u8(W.T).t(), dev_u8(XS), dev_u8(WS.T).t())
    torch.cuda.synchronize()
    Y, S = oracle.gemm_mxfp8(X, W, XS, WS)
    assert oracle.max_normalized_error(y.cpu().numpy(), Y, S) <= TOL


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (5, 48, 32), (130, 272, 1040), (1024, 4096, 4096)])
def test_wt_int8_exact(M, N, K):
    """int8 with W as [N, K] rows: the [K, N] call's bytes, and the exact integer product."""
    X, W = int_i8(50, (M, K)), int_i8(51, (K, N))
    xd = torch.from_numpy(X).to(DEV)
    a = bg.mm(xd, torch.from_numpy(W).to(DEV))
    b = bg.mm(xd, torch.from_numpy(np.ascontiguousarray(W.T)).to(DEV).t())
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if M * N * K <= 1 << 26:
        assert np.array_equal(b.cpu().numpy().astype(np.int64), X.astype(np.int64) @ W.astype(np.int64))


def _padded(a, pad):
    """Device copy of a 2-D numpy array in rows of a.shape[1] + pad elements (a view of the logical part)."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                         else np.ascontiguousarray(a))
    buf = torch.zeros((a.shape[0], a.shape[1] + pad), dtype=t.dtype)
    buf[:, :a.shape[1]] = t
    return buf.to(DEV)[:, :a.shape[1]]


@pytest.mark.parametrize("family", ["bf16", "mx", "i8"])
def test_wt_random_shapes_and_padding(family):
    """40 seeded random shapes per family (ragged in M, N and K) with random row padding of X, W^T,
    Y and the scales: the [N, K] call's bytes equal the [K, N] call's."""
    rng = np.random.default_rng({"bf16": 11, "mx": 12, "i8": 13}[family])
    kq, nq = {"bf16": (8, 8), "mx": (32, 16), "i8": (16, 16)}[family]
    ypad = 4  # fp32 / int32 output rows stay 16-byte aligned
    for case in range(40):
        M = int(rng.integers(1, 300))
        N = nq * int(rng.integers(1, 640 // nq))
        K = kq * int(rng.integers(1, 1100 // kq))
        pad = int(rng.choice([0, 16, 48]))   # keeps every row 16-byte aligned for 1- and 2-byte elements
        if family == "bf16":
            X, W = normal_bf16(100 + case, (M, K)), normal_bf16(200 + case, (K, N))
            args_kn, args_nk = (), ()
        elif family == "mx":
            X, W, XS, WS = _mx_case(M, N, K, seed=case)
            spad = int(rng.choice([0, 3, 16]))
            xs = _padded(XS, spad)
            args_kn = (xs, _padded(WS, spad))
            args_nk = (xs, _padded(WS.T, spad).t())
        else:
            X, W = int_i8(300 + case, (M, K)), int_i8(400 + case, (K, N))
            args_kn, args_nk = (), ()
        xd = _padded(X, pad)
        w_kn = _padded(W, pad)
        w_nk = _padded(W.T, pad).t()
        odt = torch.int32 if family == "i8" else torch.float32
        ya = torch.full((M, N + ypad), -1, dtype=odt, device=DEV)
        yb = torch.full((M, N + ypad), -1, dtype=odt, device=DEV)
        bg.mm(xd, w_kn, *args_kn, out=ya[:, :N])
        bg.mm(xd, w_nk, *args_nk, out=yb[:, :N])
        torch.cuda.synchronize()
        assert torch.equal(_bits(ya) if odt == torch.float32 else ya, _bits(yb) if odt == torch.float32 else yb), \
            (family, case, M, N, K, pad)
