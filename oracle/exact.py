"""Exact brute force for tiny shapes — TEST INFRASTRUCTURE ONLY.

Pure Python, independent of ``oracle.c``: operands are decoded here from the
format definitions, products are formed exactly, and sums are taken either as
exact rationals (``fractions.Fraction``) or as the correctly rounded binary64
value of the exact sum (``math.fsum``). Used to pin the C oracle on small
inputs (the blog's matrix-multiplication definition C_ij = sum_k A_ik B_kj).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def bf16_value(bits: int) -> float:
    """bf16 bits are the high half of a binary32."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e4m3_value(code: int) -> float:
    """OCP E4M3FN: sign, 4-bit exponent (bias 7), 3-bit mantissa; S.1111.111 = NaN; no infinities."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(code: int) -> float:
    """E8M0: 2^(code-127); 0xFF = NaN."""
    code = int(code) & 0xFF
    if code == 0xFF:
        return float("nan")
    return math.ldexp(1.0, code - 127)


def f16_value(bits: int) -> float:
    """IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit mantissa; field 31 is inf / NaN."""
    bits = int(bits) & 0xFFFF
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0x1F:
        return float("nan") if m else sign * float("inf")
    if e == 0:
        return sign * (m / 1024.0) * 2.0 ** (-14)
    return sign * (1.0 + m / 1024.0) * 2.0 ** (e - 15)


def fsum_gemm_f16(X, W):
    """Correctly rounded binary64 of the exact sums for fp16 bit patterns (products exact)."""
    X = np.asarray(X)
    W = np.asarray(W)
    M, K = X.shape
    N = W.shape[1]
    Y = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    for i in range(M):
        for j in range(N):
            p = [f16_value(X[i, k]) * f16_value(W[k, j]) for k in range(K)]
            Y[i, j] = math.fsum(p)
            S[i, j] = math.fsum(abs(v) for v in p)
    return Y, S


def _products_bf16(X, W, i, j):
    K = X.shape[1]
    return [bf16_value(X[i, k]) * bf16_value(W[k, j]) for k in range(K)]  # exact in binary64


def _products_mx(X, W, XS, WS, i, j):
    K = X.shape[1]
    out = []
    for k in range(K):
        a = e4m3_value(X[i, k]) * e8m0_value(XS[i, k // 32])
        b = e4m3_value(W[k, j]) * e8m0_value(WS[k // 32, j])
        out.append(a * b)  # exact in binary64: <= 8 significant bits, exponent in range
    return out


def fsum_gemm_bf16(X, W, rows=None):
    """Correctly rounded binary64 of the exact sum, for the requested rows (default all)."""
    X = np.asarray(X)
    W = np.asarray(W)
    rows = range(X.shape[0]) if rows is None else rows
    N = W.shape[1]
    Y = np.empty((len(rows), N), dtype=np.float64)
    S = np.empty((len(rows), N), dtype=np.float64)
    for r, i in enumerate(rows):
        for j in range(N):
            p = _products_bf16(X, W, i, j)
            Y[r, j] = math.fsum(p)
            S[r, j] = math.fsum(abs(v) for v in p)
    return Y, S


def fraction_gemm_bf16(X, W):
    """Exact rational result (list of lists of Fraction)."""
    X = np.asarray(X)
    W = np.asarray(W)
    M, K = X.shape
    N = W.shape[1]
    return [[sum((Fraction(v) for v in _products_bf16(X, W, i, j)), Fraction(0)) for j in range(N)]
            for i in range(M)]


def fsum_gemm_mxfp8(X, W, XS, WS, rows=None):
    X = np.asarray(X)
    W = np.asarray(W)
    rows = range(X.shape[0]) if rows is None else rows
    N = W.shape[1]
    Y = np.empty((len(rows), N), dtype=np.float64)
    S = np.empty((len(rows), N), dtype=np.float64)
    for r, i in enumerate(rows):
        for j in range(N):
            p = _products_mx(X, W, XS, WS, i, j)
            Y[r, j] = math.fsum(p)
            S[r, j] = math.fsum(abs(v) for v in p)
    return Y, S
