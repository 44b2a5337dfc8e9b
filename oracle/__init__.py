"""CPU oracle for the batch-invariant GEMM — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It never touches a GPU and shares no
code with the HIP path: the arithmetic lives in ``oracle.c`` (plain C built
with gcc, loaded here through ctypes) and in ``exact.py`` (pure-Python exact
sums for tiny shapes).

What it computes (the nondeterminism blog, section on batch-invariant matrix
multiplication: C_ij = sum_k A_ik B_kj) and how closely the GPU must agree:

* ``gemm_bf16`` / ``gemm_f16`` / ``gemm_mxfp8`` return the fp64-accumulated
  product of the exactly decoded operands, summed with k ascending, and
  S_ij = sum_k |x_ik w_kj|. ``gemm_i8`` returns the exact int64 product.
* ``attention`` is causal softmax attention of query tokens over the keys
  and values of their sequences (section on batch-invariant attention), in
  fp64; ``attention_tol`` bounds the fp32 evaluation's error for each
  (token, head) relative to S = sum_j w_j |v_j| / sum_j w_j.
* ``max_normalized_error`` is the parity metric: max_ij |y_gpu - y| / S_ij
  (elements with S_ij = 0 must be exactly 0). Any fp32 accumulation of the
  exact products, in any order, satisfies e <= gamma_{K-1}(fp32) by the blog's
  sequential-sum bound (section on unit roundoff); the gate is 2e-3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

PARITY_TOL = 2e-3  # max normalised error allowed for bf16/MXFP8 inputs with fp32 accumulation
# bf16 output: the fp32 result is rounded once to 8 significant bits, adding at
# most u_bf16 = 2^-8 of |y| <= S(1 + gamma) to the accumulation error.
PARITY_TOL_BF16_OUT = PARITY_TOL + 2.0 ** -8 * (1 + PARITY_TOL)

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True, src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile an oracle C source into a shared library with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_e4m3.restype = ctypes.c_double
        lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_e8m0.restype = ctypes.c_double
        lib.oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_gemm_f16.restype = ctypes.c_int
        lib.oracle_gemm_f16.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_rmsnorm_bf16.restype = ctypes.c_int
        lib.oracle_rmsnorm_bf16.argtypes = [_i64, _i64, _p, _i64, _p, ctypes.c_double, _p, _i64]
        lib.oracle_rmsnorm_f32.restype = ctypes.c_int
        lib.oracle_rmsnorm_f32.argtypes = [_i64, _i64, _p, _i64, _p, ctypes.c_double, _p, _i64]
        lib.oracle_gemm_i8.restype = ctypes.c_int
        lib.oracle_gemm_i8.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemm_f64.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_gemm_bf16.restype = ctypes.c_int
        lib.oracle_gemm_bf16.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_gemm_mxfp8.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                          _p, _i64, _p, _i64]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, ctypes.c_double,
                                         _p, _p, _p]
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = path

    def set_threads(self, n: int) -> int:
        """Set the OpenMP thread count (n <= 0 keeps it); returns the count in effect."""
        return self.lib.oracle_set_threads(int(n))

    def decode_bf16(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.oracle_decode_bf16
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def decode_e4m3(self, codes) -> np.ndarray:
        c = np.asarray(codes, dtype=np.uint8)
        f = self.lib.oracle_decode_e4m3
        return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)

    def decode_e8m0(self, codes) -> np.ndarray:
        c = np.asarray(codes, dtype=np.uint8)
        f = self.lib.oracle_decode_e8m0
        return np.array([f(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)

    def decode_f16(self, bits) -> np.ndarray:
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.oracle_decode_f16
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def gemm_f16(self, X, W, want_s: bool = True):
        """fp16 X[M,K] (uint16 bits) times fp16 W[K,N]; returns (Y, S) in fp64."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        M, K = X.shape
        K2, N = W.shape
        assert K == K2, (X.shape, W.shape)
        Y = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if want_s else None
        rc = self.lib.oracle_gemm_f16(M, N, K, _ptr(X), K, _ptr(W), N, _ptr(Y), N,
                                      _ptr(S) if want_s else None, N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f16 failed rc={rc}")
        return (Y, S) if want_s else Y

    def gemm_i8(self, X, W) -> np.ndarray:
        """int8 X[M,K] times int8 W[K,N], exact, as int64."""
        X = np.ascontiguousarray(X, dtype=np.int8)
        W = np.ascontiguousarray(W, dtype=np.int8)
        M, K = X.shape
        K2, N = W.shape
        assert K == K2, (X.shape, W.shape)
        Y = np.empty((M, N), dtype=np.int64)
        rc = self.lib.oracle_gemm_i8(M, N, K, _ptr(X), K, _ptr(W), N, _ptr(Y), N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_i8 failed rc={rc}")
        return Y

    def rmsnorm(self, X, gamma, eps: float) -> np.ndarray:
        """RMSNorm of each row of X (uint16 bf16 bits or float32) with gamma, in fp64."""
        X = np.asarray(X)
        bf16 = X.dtype == np.uint16
        dt = np.uint16 if bf16 else np.float32
        X = np.ascontiguousarray(X, dtype=dt)
        G = np.ascontiguousarray(gamma, dtype=dt)
        M, D = X.shape
        assert G.shape == (D,), (G.shape, D)
        Y = np.empty((M, D), dtype=np.float64)
        f = self.lib.oracle_rmsnorm_bf16 if bf16 else self.lib.oracle_rmsnorm_f32
        rc = f(M, D, _ptr(X), D, _ptr(G), float(eps), _ptr(Y), D)
        if rc != 0:
            raise RuntimeError(f"oracle rmsnorm failed rc={rc}")
        return Y

    def attention(self, Q, K, V, seq, pos, scale: float):
        """Causal softmax attention of query tokens over per-sequence keys/values, in fp64.

        Q [T, H, D] and K, V [nseq, maxlen, Hkv, D] are bf16 bit patterns (uint16);
        seq, pos [T] give each token's sequence and position. Returns (O, S, stats):
        O and S are [T, H, D]; stats [T, H, 3] holds (A, Mabs, R) for attention_tol."""
        Q = np.ascontiguousarray(Q, dtype=np.uint16)
        K = np.ascontiguousarray(K, dtype=np.uint16)
        V = np.ascontiguousarray(V, dtype=np.uint16)
        seq = np.ascontiguousarray(seq, dtype=np.int32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, H, D = Q.shape
        nseq, maxlen, Hkv, D2 = K.shape
        assert D == D2 and V.shape == K.shape and seq.shape == (T,) and pos.shape == (T,)
        O = np.empty((T, H, D), dtype=np.float64)
        S = np.empty((T, H, D), dtype=np.float64)
        st = np.empty((T, H, 3), dtype=np.float64)
        rc = self.lib.oracle_attention(T, H, Hkv, D, nseq, maxlen, _ptr(Q), _ptr(K), _ptr(V), _ptr(seq), _ptr(pos),
                                       float(scale), _ptr(O), _ptr(S), _ptr(st))
        if rc != 0:
            raise RuntimeError(f"oracle_attention failed rc={rc}")
        return O, S, st

    def gemm_f64(self, A, B, want_s: bool = True):
        """fp64 product of fp64 operands (the oracle's accumulation core)."""
        A = np.ascontiguousarray(A, dtype=np.float64)
        B = np.ascontiguousarray(B, dtype=np.float64)
        M, K = A.shape
        K2, N = B.shape
        assert K == K2, (A.shape, B.shape)
        Y = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if want_s else None
        rc = self.lib.oracle_gemm_f64(M, N, K, _ptr(A), K, _ptr(B), N, _ptr(Y), N,
                                      _ptr(S) if want_s else None, N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f64 failed rc={rc}")
        return (Y, S) if want_s else Y

    def gemm_bf16(self, X, W, want_s: bool = True):
        """bf16 X[M,K] (uint16 bits) times bf16 W[K,N]; returns (Y, S) in fp64."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        M, K = X.shape
        K2, N = W.shape
        assert K == K2, (X.shape, W.shape)
        Y = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if want_s else None
        rc = self.lib.oracle_gemm_bf16(M, N, K, _ptr(X), K, _ptr(W), N, _ptr(Y), N,
                                       _ptr(S) if want_s else None, N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_bf16 failed rc={rc}")
        return (Y, S) if want_s else Y

    def gemm_mxfp8(self, X, W, XS, WS, want_s: bool = True):
        """MXFP8: E4M3 codes X[M,K], W[K,N]; E8M0 scales XS[M,K/32], WS[K/32,N]."""
        X = np.ascontiguousarray(X, dtype=np.uint8)
        W = np.ascontiguousarray(W, dtype=np.uint8)
        XS = np.ascontiguousarray(XS, dtype=np.uint8)
        WS = np.ascontiguousarray(WS, dtype=np.uint8)
        M, K = X.shape
        K2, N = W.shape
        assert K == K2 and K % 32 == 0, (X.shape, W.shape)
        assert XS.shape == (M, K // 32) and WS.shape == (K // 32, N), (XS.shape, WS.shape)
        Y = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if want_s else None
        rc = self.lib.oracle_gemm_mxfp8(M, N, K, _ptr(X), K, _ptr(W), N, _ptr(XS), K // 32, _ptr(WS), N,
                                        _ptr(Y), N, _ptr(S) if want_s else None, N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_mxfp8 failed rc={rc}")
        return (Y, S) if want_s else Y


_default = None
_lock = threading.Lock()


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if no library is there)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build(force=False)
            _default = Oracle(LIB_PATH)
    return _default


def set_threads(n: int) -> int:
    return default().set_threads(n)


def decode_bf16(bits):
    return default().decode_bf16(bits)


def decode_e4m3(codes):
    return default().decode_e4m3(codes)


def decode_e8m0(codes):
    return default().decode_e8m0(codes)


def decode_f16(bits):
    return default().decode_f16(bits)


def gemm_f16(X, W, want_s: bool = True):
    return default().gemm_f16(X, W, want_s)


def gemm_i8(X, W):
    return default().gemm_i8(X, W)


def rmsnorm(X, gamma, eps: float):
    return default().rmsnorm(X, gamma, eps)


def rmsnorm_tol(D: int, bf16_out: bool) -> float:
    """Relative error bound of the fp32 RMSNorm against the exact value: the sum of D
    squares (relative error at most gamma_{D-1}(fp32), halved by the square root) plus
    a few binary32 roundings (division, eps, square root, reciprocal, two products),
    and one bf16 rounding (u = 2^-8) for a bf16 output."""
    u32 = unit_roundoff(24)
    return gamma(D - 1, u32) / 2 + 8 * u32 + (unit_roundoff(8) if bf16_out else 0.0)


def gemm_f64(A, B, want_s: bool = True):
    return default().gemm_f64(A, B, want_s)


def attention(Q, K, V, seq, pos, scale: float):
    return default().attention(Q, K, V, seq, pos, scale)


def attention_tol(stats, L, D: int, bf16_out: bool) -> np.ndarray:
    """Bound on |o_gpu - o| / S for each (token, head), for any fp32 evaluation that
    forms the scores with at most two roundings per product pair, subtracts a running
    or final maximum, exponentiates in single precision (allowing 4 ulp) and adds the
    weighted values in any order, possibly as partial sums rescaled by exp(m_s - m).

    stats = (A, Mabs, R) from ``attention``; L = context length (pos + 1), broadcast
    against stats[..., 0]. Score error: delta = gamma_{2D} A + 2u Mabs. A weight's
    relative error: eps_w = 2 delta + 2 e_exp + 2u R + 3u (its score and the maximum
    both err, two exponentials with their argument roundings, one product). Weights
    with relative errors <= eps_w move o by at most 2 eps_w (1 + eps_w) S, and the two
    sums (numerator, denominator) add gamma_{2L+4} S each; one division adds u."""
    u = unit_roundoff(24)
    st = np.asarray(stats, dtype=np.float64)
    A, Mabs, R = st[..., 0], st[..., 1], st[..., 2]
    L = np.broadcast_to(np.asarray(L, dtype=np.float64), A.shape)
    e_exp = 8 * u
    delta = gamma(2 * D, u) * A + 2 * u * Mabs
    eps_w = 2 * delta + 2 * e_exp + 2 * u * R + 3 * u
    nu = (2 * L + 4) * u
    g_sum = nu / (1 - nu)
    tol = 2 * eps_w * (1 + eps_w) + 2 * g_sum + u
    if bf16_out:
        tol = tol + unit_roundoff(8) * (1 + tol)
    return tol


def gemm_bf16(X, W, want_s: bool = True):
    return default().gemm_bf16(X, W, want_s)


def gemm_mxfp8(X, W, XS, WS, want_s: bool = True):
    return default().gemm_mxfp8(X, W, XS, WS, want_s)


# ------------------------------------------------------------------ tolerance
def unit_roundoff(p: int) -> float:
    """u = 2^-p for a p-bit significand (the blog's unit-roundoff table)."""
    return 2.0 ** (-p)


def gamma(n: int, u: float) -> float:
    """gamma_n = n u / (1 - n u), the constant of the blog's sequential-sum bound."""
    nu = n * u
    if nu >= 1.0:
        return float("inf")
    return nu / (1.0 - nu)


def normalized_error(y_test, y_ref, s_ref) -> np.ndarray:
    """Elementwise |y_test - y_ref| / S; where S == 0 the error is 0 if y_test == 0 else inf."""
    y_test = np.asarray(y_test, dtype=np.float64)
    d = np.abs(y_test - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = d / s_ref
    zero = s_ref == 0
    if zero.any():
        e = np.where(zero, np.where(y_test == 0, 0.0, np.inf), e)
    e = np.where(np.isnan(e), np.inf, e)
    return e


def max_normalized_error(y_test, y_ref, s_ref) -> float:
    e = normalized_error(y_test, y_ref, s_ref)
    return float(e.max()) if e.size else 0.0
