"""Python binding of libbigemm (the batch-invariant GEMM for MI355X / gfx950).

The functions named ``bigemm_*`` mirror the C ABI in ``include/bigemm.h``
one to one and only marshal arguments (integers for device pointers and
streams). ``mm`` is a convenience wrapper over them for torch tensors; torch
supplies device memory and the current stream, nothing else — every step of
the product runs in the HIP kernels of ``libbigemm.so``.

There is no fallback: if the library is missing or the device is not gfx950
the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "BIGEMM_OK", "BIGEMM_ERR_ARG", "BIGEMM_ERR_UNSUPPORTED", "BIGEMM_ERR_DEVICE", "BIGEMM_ERR_NOMEM",
    "BIGEMM_BF16", "BIGEMM_F32", "BIGEMM_E4M3", "BIGEMM_E8M0", "BIGEMM_F16", "BIGEMM_I8", "BIGEMM_I32",
    "BigemmError", "bigemm_desc", "library_path", "load",
    "bigemm_create", "bigemm_run", "bigemm_destroy", "bigemm_status_str", "bigemm_get_config",
    "bigemm_check_args", "bigemm_abi_version", "mm", "bigemm_create_wt", "bigemm_check_args_wt",
    "bigemm_create_split_k", "bigemm_create_split_k_wt", "bigemm_workspace_size", "bigemm_run_ws",
    "bigemm_check_args_split_k", "bigemm_run_split_k_static", "BIGEMM_ERR_SCRATCH", "STATIC_SCRATCH_BYTES",
    "bigemm_rmsnorm", "bigemm_rmsnorm_check_args", "rmsnorm",
    "bigemm_kv_layout", "bigemm_kv_cache_write", "bigemm_attn_workspace_size", "bigemm_paged_attention",
    "bigemm_paged_attention_check_args", "kv_cache_write", "paged_attention", "ATTN_SPLIT",
]

BIGEMM_OK = 0
BIGEMM_ERR_ARG = 1
BIGEMM_ERR_UNSUPPORTED = 2
BIGEMM_ERR_DEVICE = 3
BIGEMM_ERR_NOMEM = 4
BIGEMM_ERR_SCRATCH = 5
STATIC_SCRATCH_BYTES = 64 << 20  # BIGEMM_STATIC_SCRATCH_BYTES

BIGEMM_BF16 = 1
BIGEMM_F32 = 2
BIGEMM_E4M3 = 3
BIGEMM_E8M0 = 4
BIGEMM_F16 = 5
BIGEMM_I8 = 6
BIGEMM_I32 = 7

ATTN_SPLIT = 256  # BIGEMM_ATTN_SPLIT: KV positions per split of the paged attention

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbigemm.so")
_lib = None
_lock = threading.Lock()


class BigemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_str(status)} (status {status})")


class bigemm_desc(ctypes.Structure):
    _fields_ = [("x_type", ctypes.c_int32), ("w_type", ctypes.c_int32),
                ("y_type", ctypes.c_int32), ("scale_block", ctypes.c_int32)]


class bigemm_kv_layout(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libbigemm.so (built in-tree by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
        lib.bigemm_create.restype = ctypes.c_int
        lib.bigemm_create.argtypes = [ctypes.POINTER(bigemm_desc), ctypes.POINTER(vp)]
        lib.bigemm_run.restype = ctypes.c_int
        lib.bigemm_run.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
        lib.bigemm_destroy.restype = ctypes.c_int
        lib.bigemm_destroy.argtypes = [vp]
        lib.bigemm_status_str.restype = ctypes.c_char_p
        lib.bigemm_status_str.argtypes = [ctypes.c_int]
        lib.bigemm_get_config.restype = ctypes.c_int
        lib.bigemm_get_config.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.bigemm_check_args.restype = ctypes.c_int
        lib.bigemm_check_args.argtypes = [ctypes.POINTER(bigemm_desc), i64, i64, i64, vp, i64, vp, i64,
                                          vp, i64, vp, i64, vp, i64]
        lib.bigemm_create_wt.restype = ctypes.c_int
        lib.bigemm_create_wt.argtypes = [ctypes.POINTER(bigemm_desc), ctypes.POINTER(vp)]
        lib.bigemm_check_args_wt.restype = ctypes.c_int
        lib.bigemm_check_args_wt.argtypes = [ctypes.POINTER(bigemm_desc), i64, i64, i64, vp, i64, vp, i64,
                                             vp, i64, vp, i64, vp, i64]
        lib.bigemm_abi_version.restype = i32
        lib.bigemm_abi_version.argtypes = []
        lib.bigemm_rmsnorm.restype = ctypes.c_int
        lib.bigemm_rmsnorm.argtypes = [i32, i64, i64, vp, i64, vp, vp, i64, ctypes.c_float, vp]
        lib.bigemm_rmsnorm_check_args.restype = ctypes.c_int
        lib.bigemm_rmsnorm_check_args.argtypes = [i32, i64, i64, vp, i64, vp, vp, i64]
        lib.bigemm_create_split_k.restype = ctypes.c_int
        lib.bigemm_create_split_k.argtypes = [ctypes.POINTER(bigemm_desc), i32, ctypes.POINTER(vp)]
        lib.bigemm_create_split_k_wt.restype = ctypes.c_int
        lib.bigemm_create_split_k_wt.argtypes = [ctypes.POINTER(bigemm_desc), i32, ctypes.POINTER(vp)]
        lib.bigemm_workspace_size.restype = ctypes.c_int
        lib.bigemm_workspace_size.argtypes = [vp, i64, i64, i64, ctypes.POINTER(ctypes.c_uint64)]
        lib.bigemm_check_args_split_k.restype = ctypes.c_int
        lib.bigemm_check_args_split_k.argtypes = [ctypes.POINTER(bigemm_desc), i32, i64, i64, i64, vp, i64, vp, i64,
                                                  vp, i64, vp, ctypes.c_uint64]
        lib.bigemm_run_split_k_static.restype = ctypes.c_int
        lib.bigemm_run_split_k_static.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        lib.bigemm_run_ws.restype = ctypes.c_int
        lib.bigemm_run_ws.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp,
                                      ctypes.c_uint64, vp]
        kvp = ctypes.POINTER(bigemm_kv_layout)
        lib.bigemm_kv_cache_write.restype = ctypes.c_int
        lib.bigemm_kv_cache_write.argtypes = [kvp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.bigemm_attn_workspace_size.restype = ctypes.c_int
        lib.bigemm_attn_workspace_size.argtypes = [kvp, i64, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
        lib.bigemm_paged_attention.restype = ctypes.c_int
        lib.bigemm_paged_attention.argtypes = [kvp, i64, i32, i32, ctypes.c_float, i32, vp, vp, vp, vp, vp, vp, vp,
                                               vp, ctypes.c_uint64, vp]
        lib.bigemm_paged_attention_check_args.restype = ctypes.c_int
        lib.bigemm_paged_attention_check_args.argtypes = [kvp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                          ctypes.c_uint64]
        _lib = lib
        return lib


def _status_str(status: int) -> str:
    try:
        return load().bigemm_status_str(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used to format an error message
        return "unknown"


def bigemm_status_str(status: int) -> str:
    return load().bigemm_status_str(int(status)).decode()


def bigemm_abi_version() -> int:
    return int(load().bigemm_abi_version())


def _desc(x_type, w_type, y_type, scale_block):
    return bigemm_desc(int(x_type), int(w_type), int(y_type), int(scale_block))


def bigemm_create(x_type: int, w_type: int, y_type: int = BIGEMM_F32, scale_block: int = 0) -> int:
    """Create a handle on the current HIP device; returns it as an integer. Raises BigemmError."""
    h = ctypes.c_void_p()
    d = _desc(x_type, w_type, y_type, scale_block)
    st = load().bigemm_create(ctypes.byref(d), ctypes.byref(h))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_create")
    return int(h.value)


def bigemm_create_split_k(x_type: int, w_type: int, y_type: int, k_chunk: int) -> int:
    """Create an opt-in split-K handle (bf16 / fp16 inputs). Raises BigemmError."""
    h = ctypes.c_void_p()
    d = _desc(x_type, w_type, y_type, 0)
    st = load().bigemm_create_split_k(ctypes.byref(d), int(k_chunk), ctypes.byref(h))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_create_split_k")
    return int(h.value)


def bigemm_create_split_k_wt(x_type: int, w_type: int, y_type: int, k_chunk: int) -> int:
    """Create an opt-in split-K handle whose W is given as [N, K] (bf16 / fp16). Raises BigemmError."""
    h = ctypes.c_void_p()
    d = _desc(x_type, w_type, y_type, 0)
    st = load().bigemm_create_split_k_wt(ctypes.byref(d), int(k_chunk), ctypes.byref(h))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_create_split_k_wt")
    return int(h.value)


def bigemm_create_wt(x_type: int, w_type: int, y_type: int = BIGEMM_F32, scale_block: int = 0) -> int:
    """Create a handle whose W is given as [N, K] (MXFP8: W_scale [N, K/32]). Raises BigemmError."""
    h = ctypes.c_void_p()
    d = _desc(x_type, w_type, y_type, scale_block)
    st = load().bigemm_create_wt(ctypes.byref(d), ctypes.byref(h))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_create_wt")
    return int(h.value)


def bigemm_workspace_size(h: int, M: int, N: int, K: int) -> int:
    n = ctypes.c_uint64()
    st = load().bigemm_workspace_size(ctypes.c_void_p(h) if h else None, M, N, K, ctypes.byref(n))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_workspace_size")
    return int(n.value)


def bigemm_run_ws(h: int, M: int, N: int, K: int, X: int, ldx: int, W: int, ldw: int, Y: int, ldy: int,
                  X_scale: int = 0, ldxs: int = 0, W_scale: int = 0, ldws: int = 0, workspace: int = 0,
                  workspace_bytes: int = 0, stream: int = 0, check: bool = True) -> int:
    """bigemm_run with a caller-provided device workspace. Raises BigemmError unless check=False."""
    st = load().bigemm_run_ws(ctypes.c_void_p(h) if h else None, M, N, K,
                              X or None, ldx, W or None, ldw, Y or None, ldy,
                              X_scale or None, ldxs, W_scale or None, ldws,
                              workspace or None, int(workspace_bytes), stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_run_ws")
    return int(st)


def bigemm_run_split_k_static(h: int, M: int, N: int, K: int, X: int, ldx: int, W: int, ldw: int, Y: int,
                              ldy: int, stream: int = 0, check: bool = True) -> int:
    """bigemm_run_ws of a split-K handle with the library's static scratch buffer (allocates nothing).
    Raises BigemmError unless check=False."""
    st = load().bigemm_run_split_k_static(ctypes.c_void_p(h) if h else None, M, N, K, X or None, ldx,
                                          W or None, ldw, Y or None, ldy, stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_run_split_k_static")
    return int(st)


def bigemm_destroy(h: int) -> int:
    return int(load().bigemm_destroy(ctypes.c_void_p(h) if h else None))


def bigemm_run(h: int, M: int, N: int, K: int, X: int, ldx: int, W: int, ldw: int, Y: int, ldy: int,
               X_scale: int = 0, ldxs: int = 0, W_scale: int = 0, ldws: int = 0, stream: int = 0,
               check: bool = True) -> int:
    """Enqueue Y = X W (device pointers as integers). Raises BigemmError unless check=False."""
    st = (_lib or load()).bigemm_run(ctypes.c_void_p(h) if h else None, M, N, K,
                           X or None, ldx, W or None, ldw, Y or None, ldy,
                           X_scale or None, ldxs, W_scale or None, ldws, stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_run")
    return int(st)


def bigemm_get_config(h: int):
    bm, bn, bk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = load().bigemm_get_config(ctypes.c_void_p(h) if h else None, ctypes.byref(bm), ctypes.byref(bn),
                                  ctypes.byref(bk))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_get_config")
    return bm.value, bn.value, bk.value


def bigemm_check_args(x_type: int, w_type: int, y_type: int, scale_block: int, M: int, N: int, K: int,
                      X: int, ldx: int, W: int, ldw: int, Y: int, ldy: int,
                      X_scale: int = 0, ldxs: int = 0, W_scale: int = 0, ldws: int = 0) -> int:
    """The library's argument validation (pure host function); returns the status code."""
    d = _desc(x_type, w_type, y_type, scale_block)
    return int(load().bigemm_check_args(ctypes.byref(d), M, N, K, X or None, ldx, W or None, ldw,
                                        Y or None, ldy, X_scale or None, ldxs, W_scale or None, ldws))


def bigemm_check_args_wt(x_type: int, w_type: int, y_type: int, scale_block: int, M: int, N: int, K: int,
                         X: int, ldx: int, W: int, ldw: int, Y: int, ldy: int,
                         X_scale: int = 0, ldxs: int = 0, W_scale: int = 0, ldws: int = 0) -> int:
    """Argument validation of a bigemm_create_wt handle (W [N, K], ldw >= K); returns the status code."""
    d = _desc(x_type, w_type, y_type, scale_block)
    return int(load().bigemm_check_args_wt(ctypes.byref(d), M, N, K, X or None, ldx, W or None, ldw,
                                           Y or None, ldy, X_scale or None, ldxs, W_scale or None, ldws))


def bigemm_check_args_split_k(x_type: int, w_type: int, y_type: int, k_chunk: int, M: int, N: int, K: int,
                              X: int, ldx: int, W: int, ldw: int, Y: int, ldy: int, workspace: int = 0,
                              workspace_bytes: int = 0) -> int:
    """Argument validation of bigemm_run_ws on a split-K handle (pure host function); returns the status."""
    d = _desc(x_type, w_type, y_type, 0)
    return int(load().bigemm_check_args_split_k(ctypes.byref(d), int(k_chunk), M, N, K, X or None, ldx, W or None,
                                                ldw, Y or None, ldy, workspace or None, int(workspace_bytes)))


# ------------------------------------------------------------------ torch wrapper
_handles = {}


# input family -> (x/w dtype, scale block)
_FAMILIES = {"bf16": (BIGEMM_BF16, 0), "f16": (BIGEMM_F16, 0), "mx": (BIGEMM_E4M3, 32), "i8": (BIGEMM_I8, 0)}


def _handle(kind: str, device_index: int, y_type: int = BIGEMM_F32, k_chunk: int = 0, wt: bool = False) -> int:
    """One cached handle per (input family, output type, split-K chunk, W layout, device)."""
    import torch

    key = (kind, y_type, k_chunk, wt, device_index)
    h = _handles.get(key)
    if h is None:
        t, sb = _FAMILIES[kind]
        with torch.cuda.device(device_index):
            if k_chunk:
                h = (bigemm_create_split_k_wt if wt else bigemm_create_split_k)(t, t, y_type, k_chunk)
            elif wt:
                h = bigemm_create_wt(t, t, y_type, sb)
            else:
                h = bigemm_create(t, t, y_type, sb)
        _handles[key] = h
    return h


def _ld(t) -> int:
    """Leading dimension in elements (a single row's stride is arbitrary in torch; use its width)."""
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1])


def mm(x, w, x_scale=None, w_scale=None, out=None, stream=None, out_dtype=None, k_chunk=None,
       workspace=None):
    """Y = X W on the GPU through libbigemm.

    bf16: ``x`` [M, K] and ``w`` [K, N] are torch.bfloat16 (or int16/uint16 bit
    patterns). fp16: torch.float16. int8: torch.int8 (int32 output).
    MXFP8: ``x``/``w`` are torch.float8_e4m3fn (or uint8 codes) and
    ``x_scale`` [M, K/32], ``w_scale`` [K/32, N] are uint8 E8M0 bytes. Rows
    must be contiguous; the leading dimension is taken from ``stride(0)``.
    ``w`` may instead be the transpose of an [N, K] array with contiguous rows
    (``weight.t()`` of a linear layer's weight, so ``stride(0) == 1``): it then
    runs through the W-transposed handle with no copy, and the output bytes are
    those of the [K, N] layout. For MXFP8, ``w_scale`` must then be the
    transpose of an [N, K/32] array likewise.
    Output: ``out`` if given (its dtype selects the output type), else a new
    [M, N] tensor of ``out_dtype`` (float32 or bfloat16 for floating inputs,
    default float32; int32 for int8).
    ``k_chunk`` (bf16 / fp16 only) selects the opt-in split-K handle with that
    K chunk (for either layout of ``w``); its workspace is ``workspace`` (a
    CUDA tensor of at least ``bigemm_workspace_size`` bytes) or a fresh torch
    allocation.
    """
    import torch

    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    M, K = x.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    xst, wst = x.stride(), w.stride()
    # W given as the transposed view of an [N, K] array with contiguous rows.
    wt = N > 1 and wst[1] != 1 and (K == 1 or wst[0] == 1)
    if not (x.is_cuda and w.is_cuda) or (K > 1 and xst[1] != 1) or (not wt and N > 1 and wst[1] != 1):
        raise ValueError("operands must be CUDA tensors with contiguous rows")
    if x.dtype != w.dtype:
        raise ValueError(f"x and w must have one dtype ({x.dtype} vs {w.dtype})")
    mx = x_scale is not None or w_scale is not None
    if mx:
        if x.element_size() != 1:
            raise ValueError("MXFP8 operands must be 1-byte E4M3 codes")
        if x_scale is None or w_scale is None:
            raise ValueError("MXFP8 needs both x_scale and w_scale")
        kind = "mx"
    elif x.dtype == torch.float16:
        kind = "f16"
    elif x.dtype == torch.int8:
        kind = "i8"
    elif x.element_size() == 2:
        kind = "bf16"
    else:
        raise ValueError(f"unsupported operand dtype {x.dtype}")
    if out is not None:
        out_dtype = out.dtype
    elif out_dtype is None:
        out_dtype = torch.int32 if kind == "i8" else torch.float32
    ytype = _ytypes(torch).get(out_dtype)
    if ytype is None:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    dev = x.get_device()
    if out is None:
        # rows start 16-byte aligned: for a width that leaves them short, allocate padded rows
        per = 16 // torch.empty((), dtype=out_dtype).element_size()
        ldo = -(-N // per) * per
        out = torch.empty((M, ldo), dtype=out_dtype, device=x.device)[:, :N]
    ost = out.stride()
    if out.shape != (M, N) or (N > 1 and ost[1] != 1):
        raise ValueError("out must be [M, N] with contiguous rows")
    if stream is None:
        stream = _current_stream(torch, x)
    # Leading dimensions (elements). A single row's stride is arbitrary in torch and only that row is
    # addressed, so it is given as the row width rounded up to whole 16-byte units.
    ldx = xst[0] if M > 1 else _ld_width(K, x.element_size())
    if wt:   # rows of the [N, K] array w.t()
        ldw = wst[1] if N > 1 else _ld_width(K, w.element_size())
    else:
        ldw = wst[0] if K > 1 else _ld_width(N, w.element_size())
    ldy = ost[0] if M > 1 else _ld_width(N, out.element_size())
    # The handle belongs to x's device, and the library runs a handle only on its own device.
    with _on_device(torch, dev):
        if k_chunk:
            if kind not in ("bf16", "f16"):
                raise ValueError("split-K is provided for bf16 and fp16 inputs")
            h = _handle(kind, dev, ytype, int(k_chunk), wt)
            need = bigemm_workspace_size(h, M, N, K)
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
            ws_bytes = workspace.numel() * workspace.element_size()
            bigemm_run_ws(h, M, N, K, x.data_ptr(), ldx, w.data_ptr(), ldw, out.data_ptr(),
                          ldy, 0, 0, 0, 0, workspace.data_ptr(), ws_bytes, stream)
            return out
        h = _handles.get((kind, ytype, 0, wt, dev))
        if h is None:
            h = _handle(kind, dev, ytype, 0, wt)  # raises BigemmError for a combination not provided
        if mx:
            if tuple(x_scale.shape) != (M, K // 32) or tuple(w_scale.shape) != (K // 32, N):
                raise ValueError(f"scales must be [M, K/32] = [{M}, {K // 32}] and [K/32, N] = [{K // 32}, {N}]")
            ws = w_scale.t() if wt else w_scale   # rows: [N, K/32] for W^T, else [K/32, N]
            for t in (x_scale, ws):
                if not t.is_cuda or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
                    raise ValueError("scales must be 2-D CUDA tensors with contiguous rows "
                                     "(w_scale in the same layout as w)")
            bigemm_run(h, M, N, K, x.data_ptr(), ldx, w.data_ptr(), ldw, out.data_ptr(), ldy,
                       x_scale.data_ptr(), _ld(x_scale), w_scale.data_ptr(), _ld(ws), stream)
        else:
            bigemm_run(h, M, N, K, x.data_ptr(), ldx, w.data_ptr(), ldw, out.data_ptr(), ldy,
                       0, 0, 0, 0, stream)
    return out


_YTYPES = None


def _ytypes(torch):
    global _YTYPES
    if _YTYPES is None:
        _YTYPES = {torch.float32: BIGEMM_F32, torch.bfloat16: BIGEMM_BF16, torch.int32: BIGEMM_I32}
    return _YTYPES


def _ld_width(width: int, esize: int) -> int:
    """A single row's leading dimension: its width rounded up to whole 16-byte units."""
    per = 16 // esize
    return -(-int(width) // per) * per


def _current_stream(torch, t) -> int:
    """The raw current stream of t's device (the private accessor skips building a Stream object)."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return get(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


class _NoDeviceSwitch:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_NO_SWITCH = _NoDeviceSwitch()


def _on_device(torch, dev: int):
    """torch.cuda.device(dev), or nothing when dev is already the current device."""
    get = getattr(torch._C, "_cuda_getDevice", None)
    if get is not None and get() == dev:
        return _NO_SWITCH
    return torch.cuda.device(dev)


def bigemm_rmsnorm(dtype: int, M: int, D: int, X: int, ldx: int, gamma: int, Y: int, ldy: int, eps: float,
                   stream: int = 0, check: bool = True) -> int:
    """Enqueue the batch-invariant RMSNorm (device pointers as integers)."""
    st = (_lib or load()).bigemm_rmsnorm(int(dtype), M, D, X or None, ldx, gamma or None, Y or None, ldy, float(eps),
                               stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_rmsnorm")
    return int(st)


def bigemm_rmsnorm_check_args(dtype: int, M: int, D: int, X: int, ldx: int, gamma: int, Y: int, ldy: int) -> int:
    return int(load().bigemm_rmsnorm_check_args(int(dtype), M, D, X or None, ldx, gamma or None, Y or None, ldy))


def rmsnorm(x, gamma, eps: float = 1e-6, out=None, stream=None):
    """Batch-invariant RMSNorm of each row of ``x`` [M, D] with ``gamma`` [D]: bf16 (or
    int16/uint16 bf16 bit patterns) or float32, output of the same type. ``out`` may be
    ``x`` itself (in place)."""
    import torch

    if x.dim() != 2 or gamma.dim() != 1 or gamma.shape[0] != x.shape[1]:
        raise ValueError("x must be [M, D] and gamma [D]")
    if x.dtype != gamma.dtype or not x.is_cuda or not gamma.is_cuda:
        raise ValueError("x and gamma must be CUDA tensors of one dtype")
    if x.element_size() == 2:
        dtype = BIGEMM_BF16
    elif x.dtype == torch.float32:
        dtype = BIGEMM_F32
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    M, D = x.shape
    xst = x.stride()
    if (D > 1 and xst[1] != 1) or not gamma.is_contiguous():
        raise ValueError("rows must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    ost = out.stride()
    if out.shape != x.shape or out.dtype != x.dtype or (D > 1 and ost[1] != 1):
        raise ValueError("out must match x")
    if stream is None:
        stream = _current_stream(torch, x)
    ldx = xst[0] if M > 1 else D
    ldy = ost[0] if M > 1 else D
    with _on_device(torch, x.get_device()):
        bigemm_rmsnorm(dtype, M, D, x.data_ptr(), ldx, gamma.data_ptr(), out.data_ptr(), ldy, eps, stream)
    return out


# ------------------------------------------------------------------ paged attention
def bigemm_kv_cache_write(kv: bigemm_kv_layout, T: int, K_new: int, V_new: int, seq_ids: int, positions: int,
                          block_table: int, K_cache: int, V_cache: int, stream: int = 0, check: bool = True) -> int:
    """Enqueue the KV-cache write of T tokens (device pointers as integers)."""
    st = load().bigemm_kv_cache_write(ctypes.byref(kv), T, K_new or None, V_new or None, seq_ids or None,
                                      positions or None, block_table or None, K_cache or None, V_cache or None,
                                      stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_kv_cache_write")
    return int(st)


def bigemm_attn_workspace_size(kv: bigemm_kv_layout, T: int, num_heads: int, max_context: int) -> int:
    n = ctypes.c_uint64()
    st = load().bigemm_attn_workspace_size(ctypes.byref(kv), T, num_heads, max_context, ctypes.byref(n))
    if st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_attn_workspace_size")
    return int(n.value)


def bigemm_paged_attention(kv: bigemm_kv_layout, T: int, num_heads: int, max_context: int, scale: float,
                           out_dtype: int, Q: int, K_cache: int, V_cache: int, seq_ids: int, positions: int,
                           block_table: int, O: int, workspace: int, workspace_bytes: int, stream: int = 0,
                           check: bool = True) -> int:
    """Enqueue the batch-invariant paged attention (device pointers as integers)."""
    st = load().bigemm_paged_attention(ctypes.byref(kv), T, num_heads, max_context, float(scale), int(out_dtype),
                                       Q or None, K_cache or None, V_cache or None, seq_ids or None,
                                       positions or None, block_table or None, O or None, workspace or None,
                                       int(workspace_bytes), stream or None)
    if check and st != BIGEMM_OK:
        raise BigemmError(st, "bigemm_paged_attention")
    return int(st)


def bigemm_paged_attention_check_args(kv: bigemm_kv_layout, T: int, num_heads: int, max_context: int,
                                      out_dtype: int, Q: int, K_cache: int, V_cache: int, seq_ids: int,
                                      positions: int, block_table: int, O: int, workspace: int,
                                      workspace_bytes: int) -> int:
    return int(load().bigemm_paged_attention_check_args(
        ctypes.byref(kv), T, num_heads, max_context, int(out_dtype), Q or None, K_cache or None, V_cache or None,
        seq_ids or None, positions or None, block_table or None, O or None, workspace or None,
        int(workspace_bytes)))


def _kv_layout(k_cache, block_table):
    """Layout of a cache tensor [num_blocks, num_kv_heads, block_size, head_dim] and its table."""
    if k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim], block_table 2-D")
    nb, hkv, bs, d = (int(v) for v in k_cache.shape)
    return bigemm_kv_layout(hkv, d, bs, nb, int(block_table.shape[0]), int(block_table.shape[1]))


def _check_cache_args(k_cache, v_cache, block_table, seq_ids, positions):
    import torch

    for t in (k_cache, v_cache, block_table, seq_ids, positions):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("cache, table and token arrays must be contiguous CUDA tensors")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.element_size() != 2:
        raise ValueError("k_cache and v_cache must be bf16 tensors of one shape")
    for t in (block_table, seq_ids, positions):
        if t.dtype != torch.int32:
            raise ValueError("block_table, seq_ids and positions must be int32")


def kv_cache_write(k_new, v_new, k_cache, v_cache, block_table, seq_ids, positions, stream=None):
    """Write the keys/values of T new tokens (``k_new``, ``v_new`` [T, num_kv_heads, head_dim]
    bf16) into the paged caches at the slots of (``seq_ids[t]``, ``positions[t]``)."""
    import torch

    _check_cache_args(k_cache, v_cache, block_table, seq_ids, positions)
    kv = _kv_layout(k_cache, block_table)
    T = int(seq_ids.shape[0])
    want = (T, kv.num_kv_heads, kv.head_dim)
    for t in (k_new, v_new):
        if tuple(t.shape) != want or t.element_size() != 2 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"k_new and v_new must be contiguous bf16 CUDA tensors of shape {want}")
    if stream is None:
        stream = torch.cuda.current_stream(k_cache.device).cuda_stream
    with torch.cuda.device(k_cache.device):
        bigemm_kv_cache_write(kv, T, k_new.data_ptr(), v_new.data_ptr(), seq_ids.data_ptr(), positions.data_ptr(),
                              block_table.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream)


def paged_attention(q, k_cache, v_cache, block_table, seq_ids, positions, max_context=None, scale=None,
                    out=None, out_dtype=None, workspace=None, stream=None):
    """Batch-invariant attention of query tokens ``q`` [T, num_heads, head_dim] (bf16) over the
    paged caches: token t attends to positions 0..positions[t] of sequence seq_ids[t].
    ``max_context`` defaults to the table's capacity (max_blocks * block_size) — it sizes
    the grid and the workspace, never the result; ``scale`` defaults to 1/sqrt(head_dim)
    rounded to float32. Output ``out`` or a new [T, num_heads, head_dim] tensor of
    ``out_dtype`` (float32 default, or bfloat16)."""
    import math

    import torch

    _check_cache_args(k_cache, v_cache, block_table, seq_ids, positions)
    kv = _kv_layout(k_cache, block_table)
    if q.dim() != 3 or q.shape[2] != kv.head_dim or q.element_size() != 2 or not q.is_cuda \
            or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 CUDA tensor [T, num_heads, head_dim]")
    T, H = int(q.shape[0]), int(q.shape[1])
    if int(seq_ids.shape[0]) != T or int(positions.shape[0]) != T:
        raise ValueError("seq_ids and positions must have one entry per query token")
    if max_context is None:
        max_context = kv.max_blocks * kv.block_size
    if scale is None:
        import numpy as np
        scale = float(np.float32(1.0 / math.sqrt(kv.head_dim)))
    if out is not None:
        out_dtype = out.dtype
    elif out_dtype is None:
        out_dtype = torch.float32
    otypes = {torch.float32: BIGEMM_F32, torch.bfloat16: BIGEMM_BF16}
    if out_dtype not in otypes:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = torch.empty((T, H, kv.head_dim), dtype=out_dtype, device=q.device)
    if tuple(out.shape) != (T, H, kv.head_dim) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, num_heads, head_dim] tensor")
    need = bigemm_attn_workspace_size(kv, T, H, int(max_context))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        bigemm_paged_attention(kv, T, H, int(max_context), scale, otypes[out_dtype], q.data_ptr(),
                               k_cache.data_ptr(), v_cache.data_ptr(), seq_ids.data_ptr(), positions.data_ptr(),
                               block_table.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes, stream)
    return out
