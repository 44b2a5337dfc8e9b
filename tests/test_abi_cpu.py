"""The C-ABI library loads, exports every declared entry point, and validates
arguments as its header states (host-only calls; no GPU needed)."""
import ctypes
import os
import re

import pytest

import invariant_gemm_deterministic_amd as bg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bigemm.h")
A = 1 << 20  # a 16-byte-aligned fake device address; check_args never dereferences pointers


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"BIGEMM_API\s+[\w\s\*]+?\b(bigemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ("bigemm_create", "bigemm_run", "bigemm_destroy", "bigemm_status_str",
                 "bigemm_get_config", "bigemm_check_args", "bigemm_abi_version",
                 "bigemm_create_split_k", "bigemm_workspace_size", "bigemm_run_ws",
                 "bigemm_rmsnorm", "bigemm_rmsnorm_check_args", "bigemm_kv_cache_write",
                 "bigemm_attn_workspace_size", "bigemm_paged_attention", "bigemm_paged_attention_check_args",
                 "bigemm_create_wt", "bigemm_check_args_wt", "bigemm_create_split_k_wt",
                 "bigemm_check_args_split_k"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bg.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert bg.bigemm_abi_version() == 8
    for s in range(6):
        assert bg.bigemm_status_str(s)
    assert "unknown" in bg.bigemm_status_str(99)


def test_null_handle_paths():
    lib = bg.load()
    assert lib.bigemm_destroy(None) == bg.BIGEMM_OK
    assert bg.bigemm_run(0, 1, 8, 8, A, 8, A, 8, A, 8, check=False) == bg.BIGEMM_ERR_ARG
    assert lib.bigemm_get_config(None, None, None, None) == bg.BIGEMM_ERR_ARG
    assert lib.bigemm_create(None, None) == bg.BIGEMM_ERR_ARG
    assert lib.bigemm_create_split_k(None, 512, None) == bg.BIGEMM_ERR_ARG
    assert lib.bigemm_create_wt(None, None) == bg.BIGEMM_ERR_ARG
    assert lib.bigemm_create_split_k_wt(None, 512, None) == bg.BIGEMM_ERR_ARG
    h = ctypes.c_void_p(1)
    assert lib.bigemm_create_wt(None, ctypes.byref(h)) == bg.BIGEMM_ERR_ARG and h.value is None
    assert lib.bigemm_check_args_wt(None, 1, 8, 8, A, 8, A, 8, A, 8, None, 0, None, 0) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_run_ws(0, 1, 8, 8, A, 8, A, 8, A, 8, check=False) == bg.BIGEMM_ERR_ARG
    n = ctypes.c_uint64()
    assert lib.bigemm_workspace_size(None, 1, 8, 8, ctypes.byref(n)) == bg.BIGEMM_ERR_ARG


BF = (bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F32, 0)
MX = (bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 32)


def chk(desc, M, N, K, X=A, ldx=None, W=A, ldw=None, Y=A, ldy=None, XS=0, ldxs=0, WS=0, ldws=0):
    return bg.bigemm_check_args(*desc, M, N, K, X, K if ldx is None else ldx, W, N if ldw is None else ldw,
                                Y, N if ldy is None else ldy, XS, ldxs, WS, ldws)


def test_check_args_accepts_valid_bf16():
    assert chk(BF, 4096, 4096, 4096) == bg.BIGEMM_OK
    # any K and N once every row is 16-byte aligned (padded rows)
    assert chk(BF, 4, 129, 4099, ldx=4104, ldw=136, ldy=132) == bg.BIGEMM_OK
    assert chk(BF, 4, 1, 1, ldx=8, ldw=8, ldy=4) == bg.BIGEMM_OK
    assert chk(BF, 4, 7, 7, ldx=8, ldw=8, ldy=8) == bg.BIGEMM_OK
    assert chk(BF, 1, 128, 256) == bg.BIGEMM_OK
    assert chk(BF, 0, 128, 256, X=0, W=0, Y=0) == bg.BIGEMM_OK       # M = 0 is a no-op
    assert chk(BF, 5, 16, 8, ldx=64, ldw=32, ldy=20) == bg.BIGEMM_OK  # padded leading dims


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=0), dict(K=0),                                    # shape rules
    dict(K=12), dict(N=12),                                              # unpadded rows of 24 bytes
    dict(ldx=4), dict(ldw=4), dict(ldy=4),                               # ld < row width
    dict(ldx=12, K=8), dict(ldy=10),                                     # rows not 16-byte aligned
    dict(X=0), dict(W=0), dict(Y=0), dict(X=A + 2), dict(Y=A + 4),      # null / misaligned
    dict(XS=A, ldxs=1),                                                  # scales on a bf16 handle
    dict(ldx=(1 << 23)),                                                 # 128*ldx*2 >= 2^31
])
def test_check_args_rejects_bf16(kw):
    base = dict(M=16, N=64, K=64)
    base.update(kw)
    M, N, K = base.pop("M"), base.pop("N"), base.pop("K")
    assert chk(BF, M, N, K, **base) == bg.BIGEMM_ERR_ARG


def test_check_args_mxfp8():
    ok = dict(XS=A, ldxs=4, WS=A, ldws=64)
    assert chk(MX, 16, 64, 128, **ok) == bg.BIGEMM_OK
    assert chk(MX, 16, 64, 160, XS=A, ldxs=5, WS=A, ldws=64) == bg.BIGEMM_OK   # K % 128 != 0 is fine
    assert chk(MX, 16, 64, 100, **ok) == bg.BIGEMM_ERR_ARG                     # K % 32 != 0
    assert chk(MX, 16, 72, 128, XS=A, ldxs=4, WS=A, ldws=72) == bg.BIGEMM_ERR_ARG  # N % 16 != 0
    assert chk(MX, 16, 64, 128, XS=0, ldxs=4, WS=A, ldws=64) == bg.BIGEMM_ERR_ARG
    assert chk(MX, 16, 64, 128, XS=A, ldxs=3, WS=A, ldws=64) == bg.BIGEMM_ERR_ARG  # ldxs < K/32
    assert chk(MX, 16, 64, 128, XS=A + 1, ldxs=4, WS=A + 3, ldws=64) == bg.BIGEMM_OK  # scales unaligned ok


def test_check_args_rejects_unsupported_descriptors():
    assert chk((bg.BIGEMM_BF16, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_BF16, bg.BIGEMM_F16, bg.BIGEMM_F32, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_I32, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F16, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 16), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_I8, bg.BIGEMM_I8, bg.BIGEMM_F32, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk((bg.BIGEMM_I8, bg.BIGEMM_I8, bg.BIGEMM_I32, 32), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED


F16 = (bg.BIGEMM_F16, bg.BIGEMM_F16, bg.BIGEMM_F32, 0)
BF_OUT_BF = (bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_BF16, 0)
I8 = (bg.BIGEMM_I8, bg.BIGEMM_I8, bg.BIGEMM_I32, 0)


def test_check_args_other_types():
    # fp16 inputs follow the bf16 rules
    assert chk(F16, 16, 64, 64) == bg.BIGEMM_OK
    assert chk(F16, 16, 64, 12) == bg.BIGEMM_ERR_ARG
    # bf16 output: rows of ldy * 2 bytes must be 16-byte aligned
    assert chk(BF_OUT_BF, 16, 64, 64) == bg.BIGEMM_OK
    assert chk(BF_OUT_BF, 16, 8, 64, ldy=8) == bg.BIGEMM_OK
    assert chk(BF_OUT_BF, 16, 8, 64, ldy=12) == bg.BIGEMM_ERR_ARG
    assert chk((bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_BF16, 32), 16, 64, 128,
               XS=A, ldxs=4, WS=A, ldws=64) == bg.BIGEMM_OK
    # int8: K and N multiples of 16, int32 rows 16-byte aligned, no scales
    assert chk(I8, 16, 64, 64) == bg.BIGEMM_OK
    assert chk(I8, 16, 64, 24) == bg.BIGEMM_ERR_ARG
    assert chk(I8, 16, 40, 64) == bg.BIGEMM_ERR_ARG
    assert chk(I8, 16, 64, 64, ldy=66) == bg.BIGEMM_ERR_ARG
    assert chk(I8, 16, 64, 64, XS=A, ldxs=2) == bg.BIGEMM_ERR_ARG


def chk_wt(desc, M, N, K, X=A, ldx=None, W=A, ldw=None, Y=A, ldy=None, XS=0, ldxs=0, WS=0, ldws=0):
    return bg.bigemm_check_args_wt(*desc, M, N, K, X, K if ldx is None else ldx,
                                   W, K if ldw is None else ldw, Y, N if ldy is None else ldy,
                                   XS, ldxs, WS, ldws)


def test_check_args_w_transposed():
    # W is [N, K]: its leading dimension is checked against K, not N
    assert chk_wt(BF, 4096, 4096, 4096) == bg.BIGEMM_OK
    assert chk_wt(BF, 16, 64, 256) == bg.BIGEMM_OK                       # ldw = K
    assert chk(BF, 16, 512, 256, ldw=256) == bg.BIGEMM_ERR_ARG          # the same ldw is short for [K, N]
    assert chk_wt(BF, 16, 512, 256, ldw=256) == bg.BIGEMM_OK
    assert chk_wt(BF, 16, 64, 256, ldw=64) == bg.BIGEMM_ERR_ARG          # ldw < K
    assert chk_wt(BF, 16, 64, 256, ldw=264) == bg.BIGEMM_OK              # padded rows
    assert chk_wt(BF, 16, 64, 256, ldw=260) == bg.BIGEMM_ERR_ARG         # rows not 16-byte aligned
    assert chk_wt(BF, 16, 64, 256, ldw=(1 << 23) - 8) == bg.BIGEMM_OK    # 128 * ldw * 2 just below 2^31
    assert chk_wt(BF, 16, 64, 256, ldw=1 << 23) == bg.BIGEMM_ERR_ARG
    assert chk_wt(BF, 16, 64, 12) == bg.BIGEMM_ERR_ARG                   # rows of 12 elements: 24 bytes
    assert chk_wt(BF, 16, 64, 12, ldx=16, ldw=16) == bg.BIGEMM_OK        # K = 12 in padded rows
    assert chk_wt(BF, 16, 12, 64) == bg.BIGEMM_OK                        # any N (Y rows of 48 bytes)
    assert chk_wt(BF, 16, 64, 64, W=A + 2) == bg.BIGEMM_ERR_ARG
    assert chk_wt(BF, 0, 64, 64, X=0, W=0, Y=0) == bg.BIGEMM_OK
    assert chk_wt(F16, 16, 64, 64) == bg.BIGEMM_OK
    assert chk_wt(BF_OUT_BF, 16, 64, 64) == bg.BIGEMM_OK
    assert chk_wt(BF, 16, 64, 64, XS=A, ldxs=2) == bg.BIGEMM_ERR_ARG        # no scales for bf16
    # int8: the same rules with ldw >= K
    assert chk_wt(I8, 16, 64, 64) == bg.BIGEMM_OK
    assert chk_wt(I8, 16, 64, 64, ldw=48) == bg.BIGEMM_ERR_ARG
    # MXFP8: W_scale is [N, K/32], so ldws is checked against K/32 and 128 * ldws < 2^31
    ok = dict(XS=A, ldxs=4, WS=A, ldws=4)
    assert chk_wt(MX, 16, 64, 128, **ok) == bg.BIGEMM_OK
    assert chk(MX, 16, 64, 128, ldw=64, **ok) == bg.BIGEMM_ERR_ARG           # ldws = 4 < N for [K, N]
    assert chk_wt(MX, 16, 64, 128, XS=A, ldxs=4, WS=A, ldws=3) == bg.BIGEMM_ERR_ARG
    assert chk_wt(MX, 16, 64, 128, XS=A, ldxs=4, WS=A + 1, ldws=5) == bg.BIGEMM_OK   # scales unaligned ok
    assert chk_wt(MX, 16, 64, 128, XS=A, ldxs=4, WS=A, ldws=(1 << 24) - 1) == bg.BIGEMM_OK
    assert chk_wt(MX, 16, 64, 128, XS=A, ldxs=4, WS=A, ldws=1 << 24) == bg.BIGEMM_ERR_ARG
    assert chk_wt(MX, 16, 64, 128, ldw=112, **ok) == bg.BIGEMM_ERR_ARG      # ldw < K
    assert chk_wt(MX, 16, 64, 128, XS=A, ldxs=4, WS=0, ldws=4) == bg.BIGEMM_ERR_ARG
    # descriptors that are not provided at all
    assert chk_wt((bg.BIGEMM_BF16, bg.BIGEMM_F16, bg.BIGEMM_F32, 0), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED
    assert chk_wt((bg.BIGEMM_E4M3, bg.BIGEMM_E4M3, bg.BIGEMM_F32, 16), 4, 64, 64) == bg.BIGEMM_ERR_UNSUPPORTED


def test_rmsnorm_check_args():
    ok = bg.bigemm_rmsnorm_check_args
    assert ok(bg.BIGEMM_BF16, 16, 4096, A, 4096, A, A, 4096) == bg.BIGEMM_OK
    assert ok(bg.BIGEMM_F32, 16, 8, A, 8, A, A, 12) == bg.BIGEMM_OK          # padded fp32 rows
    assert ok(bg.BIGEMM_BF16, 0, 64, 0, 64, 0, 0, 64) == bg.BIGEMM_OK        # M = 0 is a no-op
    assert ok(bg.BIGEMM_BF16, 16, 12, A, 16, A, A, 16) == bg.BIGEMM_ERR_ARG  # D % 8
    assert ok(bg.BIGEMM_BF16, 16, 65544, A, 65544, A, A, 65544) == bg.BIGEMM_ERR_ARG  # D > 65536
    assert ok(bg.BIGEMM_BF16, 16, 64, A, 60, A, A, 64) == bg.BIGEMM_ERR_ARG  # ldx < D
    assert ok(bg.BIGEMM_BF16, 16, 64, A, 68, A, A, 64) == bg.BIGEMM_ERR_ARG  # row not 16-byte aligned
    assert ok(bg.BIGEMM_BF16, 16, 64, A + 2, 64, A, A, 64) == bg.BIGEMM_ERR_ARG
    assert ok(bg.BIGEMM_BF16, 16, 64, A, 64, 0, A, 64) == bg.BIGEMM_ERR_ARG
    assert ok(bg.BIGEMM_E4M3, 16, 64, A, 64, A, A, 64) == bg.BIGEMM_ERR_UNSUPPORTED


def _kv(**kw):
    f = dict(num_kv_heads=2, head_dim=128, block_size=32, num_blocks=10, num_seqs=2, max_blocks=4)
    f.update(kw)
    return bg.bigemm_kv_layout(*(f[k] for k in ("num_kv_heads", "head_dim", "block_size", "num_blocks", "num_seqs",
                                                "max_blocks")))


def achk(kv=None, T=3, H=4, mc=128, odt=bg.BIGEMM_F32, Q=A, K=A, V=A, s=A, p=A, bt=A, O=A, ws=A, wsb=1 << 30):
    return bg.bigemm_paged_attention_check_args(kv or _kv(), T, H, mc, odt, Q, K, V, s, p, bt, O, ws, wsb)


def test_paged_attention_check_args():
    OK, ARG = bg.BIGEMM_OK, bg.BIGEMM_ERR_ARG
    assert achk() == OK
    assert achk(odt=bg.BIGEMM_BF16) == OK
    assert achk(T=0, Q=0, K=0, V=0, s=0, p=0, bt=0, O=0, ws=0, wsb=0) == OK
    for H in (2, 6, 8, 10, 14, 16, 30, 32):  # groups of 1 to 16 query heads per KV head
        assert achk(H=H) == OK, H
    for H in (0, 3, 34, 64):  # not a multiple of 2 KV heads, or a group of 17 or 32
        assert achk(H=H) == ARG, H
    assert achk(kv=_kv(head_dim=64)) == OK and achk(kv=_kv(head_dim=96)) == ARG
    for bs, ok in ((1, OK), (4096, OK), (24, ARG), (0, ARG), (8192, ARG)):
        assert achk(kv=_kv(block_size=bs), mc=1) == ok, bs
    for f in ("num_kv_heads", "num_blocks", "num_seqs", "max_blocks"):
        assert achk(kv=_kv(**{f: 0})) == ARG, f
    assert achk(mc=0) == ARG and achk(mc=129) == ARG and achk(mc=1) == OK  # capacity 4 * 32
    assert achk(T=-1) == ARG
    assert achk(odt=bg.BIGEMM_I32) == bg.BIGEMM_ERR_UNSUPPORTED
    for name in ("Q", "K", "V", "O", "ws"):
        assert achk(**{name: A + 4}) == ARG, name
        assert achk(**{name: 0}) == ARG, name
    for name in ("s", "p", "bt"):
        assert achk(**{name: A + 4}) == OK and achk(**{name: A + 2}) == ARG and achk(**{name: 0}) == ARG, name
    need = bg.bigemm_attn_workspace_size(_kv(), 3, 4, 128)
    assert need == 3 * 4 * 1 * 130 * 4
    assert achk(wsb=need) == OK and achk(wsb=need - 1) == ARG
    assert bg.bigemm_attn_workspace_size(_kv(max_blocks=40), 5, 8, 1280) == 5 * 8 * 5 * 130 * 4
    assert bg.bigemm_attn_workspace_size(_kv(max_blocks=41), 5, 8, 1281) == 5 * 8 * 6 * 130 * 4
    assert bg.load().bigemm_kv_cache_write(None, 1, None, None, None, None, None, None, None, None) == ARG


def test_attention_binding_rejects_host_tensors():
    """The torch wrappers validate before any device call: host tensors, wrong dtypes
    and wrong shapes raise ValueError."""
    import torch
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    s = torch.zeros(1, dtype=torch.int32)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bg.paged_attention(q, kc, kc, bt, s, s)
    with pytest.raises(ValueError):
        bg.kv_cache_write(q[:, :2], q[:, :2], kc, kc, bt, s, s)
    with pytest.raises(ValueError):
        bg.rmsnorm(torch.zeros((2, 64)), torch.zeros(64))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and a message, before it
    imports torch or touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kind", ["mxfp8", "i8"])
def test_bench_profiling_kinds_need_no_sweep(kind):
    """--kind mxfp8 / i8 (profiling runs of one kernel) are refused with the sweep on: exit status 2
    with a message, before any device work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--kind", kind], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--no-sweep" in r.stderr and r.stdout == ""


def test_check_args_split_k():
    """The split-K run's own limits: workspace present, aligned and large enough, and the fp32
    chunk sums addressable through 32-bit offsets within a 128-row tile (128 * N * 4 < 2^31)
    whatever the output type; a single chunk (K <= k_chunk) needs no workspace."""
    BFO = (bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_BF16)

    def sk(M, N, K, kc=512, ws=A, wsb=None, desc=(bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_F32), ldy=None):
        need = -(-K // kc) * M * N * 4 if K > kc else 0
        return bg.bigemm_check_args_split_k(*desc, kc, M, N, K, A, K, A, N, A, N if ldy is None else ldy, ws,
                                            need if wsb is None else wsb)

    assert sk(64, 4096, 4096) == bg.BIGEMM_OK
    assert sk(64, 4096, 512, ws=0, wsb=0) == bg.BIGEMM_OK               # one chunk: no workspace needed
    assert sk(0, 4096, 4096, ws=0, wsb=0) == bg.BIGEMM_OK               # M = 0 is a no-op
    assert sk(64, 4096, 4096, ws=0) == bg.BIGEMM_ERR_ARG                # missing
    assert sk(64, 4096, 4096, ws=A + 4) == bg.BIGEMM_ERR_ARG            # misaligned
    assert sk(64, 4096, 4096, wsb=8 * 64 * 4096 * 4 - 1) == bg.BIGEMM_ERR_ARG  # one byte short
    assert sk(64, 4096, 4096, kc=100) == bg.BIGEMM_ERR_ARG              # k_chunk not a multiple of 64
    assert bg.bigemm_check_args_split_k(*MX[:3], 512, 1, 64, 1024, A, 1024, A, 64, A, 64, A, 1 << 20) == \
        bg.BIGEMM_ERR_UNSUPPORTED
    # 128 * N * 4 just below and at 2^31: with a bf16 output the caller's ldy alone would allow both
    n_ok, n_bad = (1 << 22) - 8, 1 << 22
    assert sk(1, n_ok, 1024, desc=BFO) == bg.BIGEMM_OK
    assert sk(1, n_bad, 1024, desc=BFO) == bg.BIGEMM_ERR_ARG
    assert chk((bg.BIGEMM_BF16, bg.BIGEMM_BF16, bg.BIGEMM_BF16, 0), 1, n_bad, 1024) == bg.BIGEMM_OK
    assert sk(1, n_bad, 512, desc=BFO, ws=0, wsb=0) == bg.BIGEMM_OK    # unsplit: the ordinary limits only


def test_bench_traffic_figure_follows_the_kernel_source(tmp_path, monkeypatch):
    """bench.py reports the counted HBM traffic only while the kernel source is the one the counters
    were taken on: the summary's kernel_source_sha256 must equal the source's hash, else (or when
    either file is missing) the figure is null. The committed summary carries every value it needs."""
    import hashlib
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    committed = open(bench.TRAFFIC_SUMMARY).read()
    for key in ("kernel_source_sha256=", "fetch_scale=", "write_scale=", "traffic_bytes_per_launch="):
        assert key in committed
    src = tmp_path / "kernels.hip"
    src.write_bytes(b"// one kernel source\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    summ = tmp_path / "traffic.md"
    summ.write_text(f"# summary\n\n| a | b |\n\nkernel_source_sha256={digest}\ntraffic_bytes_per_launch=470109056\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summ))
    assert bench.measured_traffic() == 470109056
    src.write_bytes(b"// the source after an edit\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
