"""Pins for the CPU oracle: checks against facts the pages and mathematics fix.

Every check takes an ``oracle.Oracle`` so that the same checks can be run on
deliberately broken copies of the oracle (tests/test_oracle_mutations.py):
each plausible mistake must make at least one of them fail.

Sources of truth used here, none of which is the oracle itself:
  * exact arithmetic (``fractions.Fraction``, ``math.fsum``) on tiny inputs;
  * integer-valued inputs, whose products and sums are exact in binary64;
  * closed forms derived from the blog's linspace experiment (section on
    batch invariance: a = linspace(-1000, 1000, 2048*4096) reshaped [2048, 4096],
    b = linspace(-1000, 1000, 4096*4096) reshaped [4096, 4096]);
  * the blog's floating-point non-associativity example (its section on
    non-associativity), which fixes the summation order;
  * the row-separability identity [A; B] C = [A C; B C] (blog, section on
    batch invariance);
  * torch's CPU float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions and
    numpy's float16 (library routines) for the decoders;
  * numpy's int64 matrix product (a library routine) for the exact int8 GEMM;
  * invariances of power-of-two block scaling (exact in binary64);
  * torch's CPU scaled_dot_product_attention in float64 with the causal mask
    (a library routine) for the attention formula of the blog's section on
    batch-invariant attention, plus its closed forms: uniform weights when
    q = 0, a single key when the position is 0, one key when its score
    dominates by hundreds, and invariance under reordering the keys.
"""
from __future__ import annotations

import functools
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import exact
from bigemm_inputs import (normal_bf16, int_bf16, linspace_bf16, normal_e4m3, int_e4m3,
                           e8m0_scales, f32_to_bf16_bits, normal_f16, int_f16, int_i8)

U64 = 2.0 ** -53
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ reference decoders (torch, CPU)
def t_bf16(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def t_e4m3(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()


def t_e8m0(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return torch.from_numpy(c).view(torch.float8_e8m0fnu).to(torch.float32).to(torch.float64).numpy()


def _close(got, want, bound, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside bound, worst excess {float((err - bound).max())}"


# ------------------------------------------------------------------------- checks
def check_sum_order(orc: oracle.Oracle):
    """The blog's (0.1 + 1e20) - 1e20 = 0 versus 0.1 + (1e20 - 1e20) = 0.1: with the
    terms as a row of A and a column of ones as B, an oracle that sums k ascending
    must reproduce the left-to-right result of each listed order."""
    with open(os.path.join(GOLDEN, "fp_nonassoc.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for r in rows:
        terms = [float(v) for v in r[:3]]
        expect = float(r[3])
        Y = orc.gemm_f64(np.array([terms]), np.ones((3, 1)), want_s=False)
        assert Y[0, 0] == expect, (terms, Y[0, 0], expect)


def check_bruteforce_bf16(orc: oracle.Oracle, trials: int = 12):
    rng = np.random.default_rng(1234)
    for t in range(trials):
        M, N, K = int(rng.integers(1, 7)), int(rng.integers(1, 7)), int(rng.integers(1, 65))
        X = normal_bf16(100 + t, (M, K))
        W = normal_bf16(200 + t, (K, N))
        Y, S = orc.gemm_bf16(X, W)
        Yf, Sf = exact.fsum_gemm_bf16(X, W)
        g = oracle.gamma(max(K - 1, 0), U64)
        _close(Y, Yf, g * Sf, f"bf16 brute force M={M} N={N} K={K}")
        _close(S, Sf, g * Sf, f"bf16 S brute force M={M} N={N} K={K}")
    # exact rationals agree with the correctly rounded fsum on one case
    X = normal_bf16(7, (2, 24))
    W = normal_bf16(8, (24, 3))
    Q = exact.fraction_gemm_bf16(X, W)
    Yf, _ = exact.fsum_gemm_bf16(X, W)
    for i in range(2):
        for j in range(3):
            assert float(Q[i][j]) == Yf[i, j]


def check_bruteforce_mx(orc: oracle.Oracle, trials: int = 8):
    rng = np.random.default_rng(4321)
    for t in range(trials):
        M, N = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        K = 32 * int(rng.integers(1, 5))
        X = normal_e4m3(300 + t, (M, K))
        W = normal_e4m3(400 + t, (K, N))
        XS = e8m0_scales(500 + t, (M, K // 32), "var")
        WS = e8m0_scales(600 + t, (K // 32, N), "var")
        Y, S = orc.gemm_mxfp8(X, W, XS, WS)
        Yf, Sf = exact.fsum_gemm_mxfp8(X, W, XS, WS)
        g = oracle.gamma(K - 1, U64)
        _close(Y, Yf, g * Sf, f"mx brute force M={M} N={N} K={K}")
        _close(S, Sf, g * Sf, f"mx S brute force M={M} N={N} K={K}")


def check_integer_bf16(orc: oracle.Oracle):
    """Integer operands: every product and partial sum is an exact integer, so the
    oracle must equal int64 arithmetic exactly. Non-square shapes expose transposes."""
    for (M, K, N, s) in [(5, 40, 19, 0), (1, 8, 3, 1), (9, 200, 7, 2), (3, 3, 11, 3)]:
        X = int_bf16(700 + s, (M, K))
        W = int_bf16(800 + s, (K, N))
        Xi = t_bf16(X).astype(np.int64)
        Wi = t_bf16(W).astype(np.int64)
        Y = orc.gemm_bf16(X, W, want_s=False)
        assert np.array_equal(Y, (Xi @ Wi).astype(np.float64)), f"integer bf16 {M}x{K}x{N}"


def check_integer_mx(orc: oracle.Oracle):
    """E4M3 integers with K-varying E8M0 scales 2^[-4, 4]: x~ * 2^4 and w~ * 2^4 are
    integers, so 256 * Y must equal an int64 product exactly."""
    for (M, K, N, s) in [(4, 96, 6, 0), (2, 256, 5, 1), (7, 32, 9, 2)]:
        X = int_e4m3(900 + s, (M, K))
        W = int_e4m3(950 + s, (K, N))
        XS = e8m0_scales(990 + s, (M, K // 32), "var")
        WS = e8m0_scales(995 + s, (K // 32, N), "var")
        xs_e = XS.astype(np.int64) - 127 + 4      # exponent + 4 >= 0
        ws_e = WS.astype(np.int64) - 127 + 4
        Xi = t_e4m3(X).astype(np.int64) * (1 << np.repeat(xs_e, 32, axis=1))
        Wi = t_e4m3(W).astype(np.int64) * (1 << np.repeat(ws_e, 32, axis=0))
        Y = orc.gemm_mxfp8(X, W, XS, WS, want_s=False)
        assert np.array_equal(Y * 256.0, (Xi @ Wi).astype(np.float64)), f"integer mx {M}x{K}x{N}"


def check_decoders(orc: oracle.Oracle):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.decode_e4m3(codes)
    ref = t_e4m3(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]) and np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    # OCP E4M3FN landmarks: 1.0, max 448, min subnormal 2^-9, min normal 2^-6, NaN at S.1111.111
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and mine[0xFE] == -448.0
    e8 = orc.decode_e8m0(codes)
    r8 = t_e8m0(codes)
    assert np.array_equal(np.isnan(e8), np.isnan(r8)) and np.array_equal(e8[:255], r8[:255])
    assert e8[127] == 1.0 and e8[0] == 2.0 ** -127 and np.isnan(e8[255])
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mb = orc.decode_bf16(allb)
    rb = t_bf16(allb)
    assert np.array_equal(np.isnan(mb), np.isnan(rb))
    okb = ~np.isnan(rb)
    assert np.array_equal(mb[okb], rb[okb]) and np.array_equal(np.signbit(mb[okb]), np.signbit(rb[okb]))


def _linspace_cols(n_total, D, cols, lo=-1000.0, hi=1000.0, dtype=np.float64):
    """Columns `cols` of linspace(lo, hi, n_total).reshape(-1, D) in fp64 (same formula as the generator)."""
    k = np.arange(n_total // D, dtype=np.float64)[:, None]
    idx = k * D + np.asarray(cols, dtype=np.float64)[None, :]
    return lo + ((hi - lo) * idx) / float(n_total - 1)


def check_linspace_closed_form(orc: oracle.Oracle):
    """Row 0 of a.b for the blog's unrounded linspace operands equals the closed form
    D a0 b0(j) + (a0 b1 + a1 b0(j)) S1 + a1 b1 S2 (exact rationals), up to the
    sequential-sum bound plus the operands' own rounding."""
    B, D = 2048, 4096
    cols = [0, 1, 2, 1000, 2047, 2048, 4094, 4095]
    a_row = (-1000.0 + (2000.0 * np.arange(D, dtype=np.float64)) / float(B * D - 1))[None, :]
    b_cols = _linspace_cols(D * D, D, cols)
    Y, S = orc.gemm_f64(a_row, b_cols)
    S1 = Fraction(D * (D - 1), 2)
    S2 = Fraction((D - 1) * D * (2 * D - 1), 6)
    a0, a1 = Fraction(-1000), Fraction(2000, B * D - 1)
    b1 = Fraction(2000 * D, D * D - 1)
    for t, j in enumerate(cols):
        b0 = Fraction(-1000) + Fraction(2000 * j, D * D - 1)
        exact_val = D * a0 * b0 + (a0 * b1 + a1 * b0) * S1 + a1 * b1 * S2
        bound = (oracle.gamma(D - 1, U64) + 8 * U64) * S[0, t]
        assert abs(Y[0, t] - float(exact_val)) <= bound, (j, Y[0, t], float(exact_val))


@functools.lru_cache(maxsize=1)
def _linspace_row0_and_cols():
    """Row 0 of the blog's bf16 linspace a [2048, 4096] and six columns of b [4096, 4096]
    (generated once per process: the full matrices are 24M elements)."""
    B, D = 2048, 4096
    a_row0 = linspace_bf16(-1000.0, 1000.0, B * D)[:D].copy()
    b = linspace_bf16(-1000.0, 1000.0, D * D, (D, D))
    cols = [0, 1, 2047, 2048, 4094, 4095]
    return a_row0, np.ascontiguousarray(b[:, cols]), cols


def check_linspace_bf16_row0(orc: oracle.Oracle):
    """bf16-rounded linspace: row 0 of a rounds to exactly -1000, so (a.b)[0, j] is
    -1000 times the exact column sum of b; the exact sums are antisymmetric,
    y[0, j] = -y[0, D-1-j], because b[k, j] = -b[D-1-k, D-1-j]."""
    D = 4096
    a_full_row0, bcols, cols = _linspace_row0_and_cols()
    assert np.all(t_bf16(a_full_row0) == -1000.0)
    Y, S = orc.gemm_bf16(a_full_row0[None, :], bcols)
    bd = t_bf16(bcols)
    sums = np.array([math.fsum(bd[:, t]) for t in range(len(cols))])
    _close(Y[0], -1000.0 * sums, oracle.gamma(D - 1, U64) * S[0], "bf16 linspace row 0")
    assert sums[0] == -sums[5] and sums[1] == -sums[4] and sums[2] == -sums[3]


def check_row_separability(orc: oracle.Oracle):
    X = normal_bf16(11, (23, 96))
    W = normal_bf16(12, (96, 40))
    Y = orc.gemm_bf16(X, W, want_s=False)
    for k in (1, 7, 16, 22):
        Yk = np.concatenate([orc.gemm_bf16(X[:k], W, want_s=False), orc.gemm_bf16(X[k:], W, want_s=False)])
        assert Yk.tobytes() == Y.tobytes(), k
    Xm = normal_e4m3(13, (9, 64))
    Wm = normal_e4m3(14, (64, 10))
    XS = e8m0_scales(15, (9, 2), "var")
    WS = e8m0_scales(16, (2, 10), "var")
    Ym = orc.gemm_mxfp8(Xm, Wm, XS, WS, want_s=False)
    for k in (1, 4, 8):
        Yk = np.concatenate([orc.gemm_mxfp8(Xm[:k], Wm, XS[:k], WS, want_s=False),
                             orc.gemm_mxfp8(Xm[k:], Wm, XS[k:], WS, want_s=False)])
        assert Yk.tobytes() == Ym.tobytes(), k


def check_mx_equals_prescaled_bf16(orc: oracle.Oracle):
    """A scaled E4M3 value is exactly representable in bf16, so the MX oracle must equal
    the bf16 oracle on operands pre-scaled elsewhere (torch decode, numpy ldexp)."""
    M, K, N = 6, 128, 7
    X = normal_e4m3(21, (M, K))
    W = normal_e4m3(22, (K, N))
    XS = e8m0_scales(23, (M, K // 32), "var")
    WS = e8m0_scales(24, (K // 32, N), "var")
    xt = np.ldexp(t_e4m3(X), np.repeat(XS.astype(np.int64) - 127, 32, axis=1))
    wt = np.ldexp(t_e4m3(W), np.repeat(WS.astype(np.int64) - 127, 32, axis=0))
    xb = f32_to_bf16_bits(xt.astype(np.float32))
    wb = f32_to_bf16_bits(wt.astype(np.float32))
    assert np.array_equal(t_bf16(xb), xt) and np.array_equal(t_bf16(wb), wt)  # exact re-encoding
    Ym = orc.gemm_mxfp8(X, W, XS, WS, want_s=False)
    Yb = orc.gemm_bf16(xb, wb, want_s=False)
    assert Ym.tobytes() == Yb.tobytes()


def check_scale_shift(orc: oracle.Oracle):
    """Moving 2^s from X's block b to W's block b leaves Y bit-identical; adding s to
    every X scale multiplies Y by exactly 2^s."""
    M, K, N = 5, 160, 6
    X = normal_e4m3(31, (M, K))
    W = normal_e4m3(32, (K, N))
    XS = e8m0_scales(33, (M, K // 32), "var")
    WS = e8m0_scales(34, (K // 32, N), "var")
    Y = orc.gemm_mxfp8(X, W, XS, WS, want_s=False)
    for b, s in [(0, 3), (2, -2), (4, 1)]:
        XS2 = XS.copy()
        WS2 = WS.copy()
        XS2[:, b] = (XS2[:, b].astype(np.int64) + s).astype(np.uint8)
        WS2[b, :] = (WS2[b, :].astype(np.int64) - s).astype(np.uint8)
        Y2 = orc.gemm_mxfp8(X, W, XS2, WS2, want_s=False)
        assert Y2.tobytes() == Y.tobytes(), (b, s)
    for s in (-3, 2):
        XS3 = (XS.astype(np.int64) + s).astype(np.uint8)
        Y3 = orc.gemm_mxfp8(X, W, XS3, WS, want_s=False)
        assert np.array_equal(Y3, np.ldexp(Y, s)), s


def check_degenerate(orc: oracle.Oracle):
    Y, S = orc.gemm_bf16(np.zeros((0, 16), np.uint16), normal_bf16(1, (16, 4)))
    assert Y.shape == (0, 4)
    Y, S = orc.gemm_bf16(np.zeros((3, 16), np.uint16), normal_bf16(1, (16, 4)))
    assert np.all(Y == 0) and np.all(S == 0)
    X = normal_bf16(2, (4, 8))
    Y = orc.gemm_bf16(X, normal_bf16(3, (8, 1)), want_s=False)
    assert Y.shape == (4, 1)


def check_decoder_f16(orc: oracle.Oracle):
    """All 65536 binary16 codes against numpy's float16 widening and against the
    pure-Python decoder written from the format definition (NaN where both say NaN)."""
    codes = np.arange(65536, dtype=np.uint16)
    got = orc.decode_f16(codes)
    lib = codes.view(np.float16).astype(np.float64)
    dfn = np.array([exact.f16_value(int(c)) for c in codes])
    for ref, name in ((lib, "numpy"), (dfn, "definition")):
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), f"fp16 decoder vs {name}: {int((~same).sum())} codes differ"
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0
    assert got[0x7C00] == np.inf and got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0


def check_bruteforce_f16(orc: oracle.Oracle, trials: int = 10):
    rng = np.random.default_rng(2468)
    for t in range(trials):
        M, N, K = int(rng.integers(1, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 65))
        X = normal_f16(1100 + t, (M, K))
        W = normal_f16(1200 + t, (K, N))
        Y, S = orc.gemm_f16(X, W)
        Yf, Sf = exact.fsum_gemm_f16(X, W)
        g = oracle.gamma(max(K - 1, 0), U64)
        _close(Y, Yf, g * Sf, f"f16 brute force M={M} N={N} K={K}")
        _close(S, Sf, g * Sf, f"f16 S brute force M={M} N={N} K={K}")


def check_integer_f16(orc: oracle.Oracle):
    """Integer binary16 operands: the oracle must equal int64 arithmetic exactly."""
    for (M, K, N, s) in [(5, 40, 19, 0), (2, 300, 3, 1), (6, 1, 7, 2)]:
        X = int_f16(1300 + s, (M, K), -64, 64)
        W = int_f16(1400 + s, (K, N), -64, 64)
        Xi = X.view(np.float16).astype(np.int64)
        Wi = W.view(np.float16).astype(np.int64)
        Y = orc.gemm_f16(X, W, want_s=False)
        assert np.array_equal(Y, (Xi @ Wi).astype(np.float64)), f"integer f16 {M}x{K}x{N}"


def check_i8(orc: oracle.Oracle):
    """int8 over the full range (-128 included): equal to numpy's int64 product, and to a
    plain Python triple loop on a tiny case; non-square shapes expose transposes."""
    for (M, K, N, s) in [(7, 96, 5, 0), (1, 16, 33, 1), (40, 512, 24, 2), (3, 3, 2, 3)]:
        X = int_i8(1500 + s, (M, K))
        W = int_i8(1600 + s, (K, N))
        Y = orc.gemm_i8(X, W)
        assert np.array_equal(Y, X.astype(np.int64) @ W.astype(np.int64)), f"i8 {M}x{K}x{N}"
    X = np.array([[-128, 127, -1], [5, -128, 0]], dtype=np.int8)
    W = np.array([[-128, 2], [127, -128], [3, 4]], dtype=np.int8)
    want = [[sum(int(X[i, k]) * int(W[k, j]) for k in range(3)) for j in range(2)] for i in range(2)]
    assert orc.gemm_i8(X, W).tolist() == want


def _py_rmsnorm(x, g, eps):
    """RMSNorm of one row in Python floats: fsum of the (exact) squares, one sqrt."""
    s = math.fsum(float(v) * float(v) for v in x)
    den = math.sqrt(s / len(x) + eps)
    return [float(v) / den * float(w) for v, w in zip(x, g)]


def check_rmsnorm_fsum(orc: oracle.Oracle):
    """Random bf16 and fp32 rows (eps 0.5 and 1e-6) against a Python evaluation of the
    blog's RMSNorm formula with a correctly rounded sum of squares."""
    rng = np.random.default_rng(97)
    for t, (D, eps) in enumerate([(8, 0.5), (24, 1e-6), (96, 1e-6), (40, 0.5)]):
        X = normal_bf16(1700 + t, (3, D))
        G = normal_bf16(1800 + t, (D,))
        Y = orc.rmsnorm(X, G, eps)
        xf, gf = t_bf16(X), t_bf16(G)
        for i in range(3):
            ref = np.array(_py_rmsnorm(xf[i], gf, eps))
            _close(Y[i], ref, 8 * U64 * np.abs(ref) + 1e-300, f"rmsnorm bf16 D={D}")
        Xf = rng.standard_normal((2, D)).astype(np.float32)
        Gf = rng.standard_normal(D).astype(np.float32)
        Yf = orc.rmsnorm(Xf, Gf, eps)
        for i in range(2):
            ref = np.array(_py_rmsnorm(Xf[i].astype(np.float64), Gf.astype(np.float64), eps))
            _close(Yf[i], ref, 8 * U64 * np.abs(ref) + 1e-300, f"rmsnorm f32 D={D}")


def check_rmsnorm_closed_forms(orc: oracle.Oracle):
    """eps = 0: a constant row c gives sign(c) * gamma exactly; scaling a row by 2^k
    leaves it bit-identical; a one-hot row a*e_p gives sign(a) * sqrt(D) * gamma_p at p
    and 0 elsewhere; rows are separable ([A; B] row by row)."""
    D = 64
    G = normal_bf16(1900, (D,))
    g = t_bf16(G)
    for c in (1.5, -0.375, 96.0):
        X = f32_to_bf16_bits(np.full((1, D), c, np.float32))
        assert np.array_equal(orc.rmsnorm(X, G, 0.0)[0], np.sign(c) * g), c
    X = normal_bf16(1901, (4, D))
    Y = orc.rmsnorm(X, G, 0.0)
    for k in (-3, 5):
        Xk = f32_to_bf16_bits(t_bf16(X).astype(np.float32) * np.float32(2.0 ** k))
        assert np.array_equal(orc.rmsnorm(Xk, G, 0.0), Y), k
    X = np.zeros((1, D), np.uint16)
    X[0, 9] = f32_to_bf16_bits(np.array([-2.5], np.float32))[0]
    Y1 = orc.rmsnorm(X, G, 0.0)[0]
    assert np.count_nonzero(Y1) == 1
    _close([Y1[9]], [-math.sqrt(D) * g[9]], 4 * U64 * abs(math.sqrt(D) * g[9]), "rmsnorm one-hot")
    A, B = normal_bf16(1902, (3, D)), normal_bf16(1903, (5, D))
    assert np.array_equal(orc.rmsnorm(np.vstack([A, B]), G, 1e-6),
                          np.vstack([orc.rmsnorm(A, G, 1e-6), orc.rmsnorm(B, G, 1e-6)]))


# ------------------------------------------------------------------ attention
def _attn_case(seed, lens, H, Hkv, D, maxlen=None):
    """Keys/values of len(lens) sequences and one query per position of each."""
    maxlen = maxlen or max(lens)
    K = normal_bf16(seed, (len(lens), maxlen, Hkv, D))
    V = normal_bf16(seed + 1, (len(lens), maxlen, Hkv, D))
    seq = np.concatenate([np.full(L, s) for s, L in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    Q = normal_bf16(seed + 2, (len(seq), H, D))
    return Q, K, V, seq, pos


def check_attention_sdpa(orc: oracle.Oracle):
    """Every position of three sequences as a query (grouped heads, H = 6 over Hkv = 2 and
    H = Hkv = 3): equal to torch's float64 scaled_dot_product_attention with the causal
    mask, keys and values repeated over each group's query heads, within 1e-12."""
    import torch.nn.functional as F
    for (H, Hkv, D, lens, seed) in [(6, 2, 24, [37, 50, 1], 2000), (3, 3, 16, [9, 20, 5], 2010)]:
        Q, K, V, seq, pos = _attn_case(seed, lens, H, Hkv, D)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        O, S, _ = orc.attention(Q, K, V, seq, pos, scale)
        off = 0
        for s_i, L in enumerate(lens):
            q = torch.from_numpy(t_bf16(Q[off:off + L])).permute(1, 0, 2)[None]
            k = torch.from_numpy(t_bf16(K[s_i, :L])).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)[None]
            v = torch.from_numpy(t_bf16(V[s_i, :L])).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)[None]
            ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)[0].permute(1, 0, 2).numpy()
            _close(O[off:off + L], ref, 1e-12 * (1 + np.abs(ref)), f"attention vs sdpa H={H} L={L}")
            absref = F.scaled_dot_product_attention(q, k, v.abs(), is_causal=True, scale=scale)[0]
            _close(S[off:off + L], absref.permute(1, 0, 2).numpy(), 1e-12 * (1 + np.abs(absref.numpy().max())),
                   "attention S vs sdpa of |v|")
            off += L


def check_attention_closed_forms(orc: oracle.Oracle):
    """q = 0: the weights are uniform, so o is the exact mean of v_0..v_p and S the mean of
    |v|, with A = Mabs = R = 0. Position 0: o = v_0. One key scoring 896 above all others
    at a score of 1024: o is that key's value exactly (exp(-896) underflows) and
    (A, Mabs, R) = (1024, 1024, 896)."""
    H, Hkv, D = 4, 2, 16
    _, K, V, _, _ = _attn_case(2100, [40], H, Hkv, D)
    pos = np.array([0, 1, 17, 39], np.int32)
    seq = np.zeros(4, np.int32)
    Q = np.zeros((4, H, D), np.uint16)
    O, S, st = orc.attention(Q, K, V, seq, pos, 0.25)
    vf = t_bf16(V[0])
    for t, p in enumerate(pos):
        for h in range(H):
            g = h // (H // Hkv)
            for e in (0, 7, 15):
                col = [Fraction(float(x)) for x in vf[:p + 1, g, e]]
                want = float(sum(col, Fraction(0)) / (p + 1))
                wabs = float(sum((abs(c) for c in col), Fraction(0)) / (p + 1))
                _close([O[t, h, e]], [want], 4 * U64 * (abs(want) + 1e-300), "mean of v")
                _close([S[t, h, e]], [wabs], 4 * U64 * wabs, "mean of |v|")
    assert not st.any(), "stats of q = 0"
    Q1 = normal_bf16(2103, (1, H, D))
    O1, S1, _ = orc.attention(Q1, K, V, np.zeros(1, np.int32), np.zeros(1, np.int32), 0.25)
    for h in range(H):
        assert np.array_equal(O1[0, h], vf[0, h // 2]) and np.array_equal(S1[0, h], np.abs(vf[0, h // 2]))
    # dominant key: q = 64 e_0, k_j = 8 e_0 except k_5 = 64 e_0; scale 1/4 gives scores 128 and 1024
    Kd = np.zeros((1, 12, Hkv, D), np.uint16)
    Kd[0, :, :, 0] = f32_to_bf16_bits(np.array([8.0], np.float32))[0]
    Kd[0, 5, :, 0] = f32_to_bf16_bits(np.array([64.0], np.float32))[0]
    Qd = np.zeros((1, H, D), np.uint16)
    Qd[0, :, 0] = f32_to_bf16_bits(np.array([64.0], np.float32))[0]
    Od, _, std = orc.attention(Qd, Kd, V[:, :12], np.zeros(1, np.int32), np.array([11], np.int32), 0.25)
    for h in range(H):
        assert np.array_equal(Od[0, h], vf[5, h // 2]), "dominant key"
    assert np.array_equal(std[0], np.tile([1024.0, 1024.0, 896.0], (H, 1))), std[0]


def check_attention_invariances(orc: oracle.Oracle):
    """Reordering the keys of a context (the same permutation on K and V) leaves the last
    position's output unchanged up to rounding; the outputs of a token do not depend on the
    other tokens or on their order (row by row); negating q negates every score, so A,
    Mabs and R are unchanged exactly; equal query heads of one group give equal outputs."""
    H, Hkv, D = 4, 2, 16
    Q, K, V, seq, pos = _attn_case(2200, [30, 30], H, Hkv, D)
    O, S, st = orc.attention(Q, K, V, seq, pos, 0.25)
    perm = np.random.default_rng(5).permutation(30)
    Kp, Vp = K.copy(), V.copy()
    Kp[0] = K[0, perm]
    Vp[0] = V[0, perm]
    last = np.array([29], np.int32)
    Op, _, _ = orc.attention(Q[29:30], Kp, Vp, np.zeros(1, np.int32), last, 0.25)
    _close(Op[0], O[29], 64 * U64 * S[29], "keys reordered")
    order = np.random.default_rng(6).permutation(len(seq))
    O2, S2, st2 = orc.attention(Q[order], K, V, seq[order], pos[order], 0.25)
    assert np.array_equal(O2, O[order]) and np.array_equal(S2, S[order]) and np.array_equal(st2, st[order])
    Qn = Q ^ np.uint16(0x8000)
    On, _, stn = orc.attention(Qn, K, V, seq, pos, 0.25)
    assert np.array_equal(stn, st), "stats under q -> -q"
    assert not np.allclose(On[pos > 3], O[pos > 3]), "negating q changes the weights"
    Qg = Q.copy()
    Qg[:, 1] = Qg[:, 0]
    Og, _, _ = orc.attention(Qg, K, V, seq, pos, 0.25)
    assert np.array_equal(Og[:, 0], Og[:, 1]) and np.array_equal(Og[:, 2:], O[:, 2:])


ALL_CHECKS = [check_sum_order, check_bruteforce_bf16, check_bruteforce_mx, check_integer_bf16,
              check_integer_mx, check_decoders, check_linspace_closed_form, check_linspace_bf16_row0,
              check_row_separability, check_mx_equals_prescaled_bf16, check_scale_shift, check_degenerate,
              check_decoder_f16, check_bruteforce_f16, check_integer_f16, check_i8,
              check_rmsnorm_fsum, check_rmsnorm_closed_forms,
              check_attention_sdpa, check_attention_closed_forms, check_attention_invariances]
