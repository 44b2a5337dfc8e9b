"""The oracle pinned to facts outside itself (see oracle_pins_lib for the sources)."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins_lib as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(orc, check):
    check(orc)


def test_unit_roundoff_table(golden_dir):
    """u = 2^-p reproduces the blog's printed table (three significant digits)."""
    import os
    with open(os.path.join(golden_dir, "unit_roundoff.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for name, p, u in rows:
        assert f"{oracle.unit_roundoff(int(p)):.2e}" == f"{float(u):.2e}", name


def test_gamma_bound_values():
    """The tolerance the parity tests use sits above gamma_{K-1}(fp32) for every K in the workloads."""
    u32 = oracle.unit_roundoff(24)
    for K in (256, 4096, 16384):
        g = oracle.gamma(K - 1, u32)
        assert g < oracle.PARITY_TOL / 2, (K, g)
    assert oracle.gamma(0, u32) == 0.0


def test_normalized_error_semantics():
    y = np.array([1.0, 0.0, 2.0])
    ref = np.array([1.0, 0.0, 1.0])
    s = np.array([2.0, 0.0, 4.0])
    e = oracle.normalized_error(y, ref, s)
    assert e.tolist() == [0.0, 0.0, 0.25]
    assert oracle.normalized_error(np.array([1e-30]), np.array([0.0]), np.array([0.0]))[0] == float("inf")
    assert oracle.normalized_error(np.array([float("nan")]), np.array([0.0]), np.array([1.0]))[0] == float("inf")


def test_attention_tol_covers_a_plain_fp32_evaluation():
    """attention_tol admits an ordinary float32 evaluation of the same attention (numpy:
    float32 scores, exp, weighted sums) and stays small enough to reject a one-position
    shift of the values (errors of order one)."""
    from bigemm_inputs import normal_bf16
    from oracle_pins_lib import t_bf16
    H, Hkv, D, L = 4, 2, 64, 300
    K = normal_bf16(2300, (1, L, Hkv, D))
    V = normal_bf16(2301, (1, L, Hkv, D))
    Q = normal_bf16(2302, (3, H, D))
    pos = np.array([0, 150, L - 1], np.int32)
    seq = np.zeros(3, np.int32)
    scale = np.float32(1.0 / np.sqrt(D))
    O, S, st = oracle.attention(Q, K, V, seq, pos, float(scale))
    tol = oracle.attention_tol(st, (pos + 1)[:, None], D, False)
    assert (tol < 2e-3).all()
    kf, vf, qf = (t_bf16(a).astype(np.float32) for a in (K[0], V[0], Q))
    for t, p in enumerate(pos):
        for h in range(H):
            g = h // (H // Hkv)
            s = (kf[:p + 1, g] @ qf[t, h]) * scale
            w = np.exp(s - s.max())
            o32 = (w @ vf[:p + 1, g]) / w.sum(dtype=np.float32)
            assert (np.abs(o32 - O[t, h]) <= tol[t, h] * S[t, h]).all(), (t, h)
            shifted = (w[:-1] @ vf[1:p + 1, g]) / w[:-1].sum() if p > 0 else vf[0, g] + 1
            assert (np.abs(shifted - O[t, h]) > tol[t, h] * S[t, h]).any(), (t, h)


def _bf16_rne(a):
    """float32 -> bfloat16 (round to nearest even, torch's CPU conversion) -> float64."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _bf16_trunc(a):
    """float32 -> bfloat16 by dropping the low 16 bits (a plausible wrong rounding) -> float64."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _rmsnorm_fp32_sequential(xf, gf, eps, D=None):
    """A plain float32 RMSNorm (the blog's formula): the squares summed left to right in
    float32 (np.cumsum keeps a float32 running sum), then mean, eps, root, reciprocal and
    two products, each rounded to float32. ``D`` replaces the divisor (a planted slip)."""
    n = np.float32(xf.shape[-1] if D is None else D)
    s = np.cumsum(xf * xf, axis=-1, dtype=np.float32)[..., -1]
    r = np.float32(1.0) / np.sqrt(s / n + np.float32(eps), dtype=np.float32)
    return (xf * r[..., None]).astype(np.float32) * gf


@pytest.mark.parametrize("D", [8, 4096, 65536])
def test_rmsnorm_tol_admits_plain_fp32_evaluations(D):
    """oracle.rmsnorm_tol (relative to |y|) admits a plain float32 RMSNorm with a sequential
    sum of squares, one with numpy's pairwise sum, and the bf16 rounding of the first, at
    D = 8, 4096 and 65536, for bf16 and float32 inputs."""
    from bigemm_inputs import normal_bf16
    from oracle_pins_lib import t_bf16
    X, G = normal_bf16(2400 + D % 97, (4, D)), normal_bf16(2401, (D,))
    rng = np.random.default_rng(D)
    Xf32 = (rng.standard_normal((3, D)) * 3).astype(np.float32)
    Gf32 = rng.standard_normal(D).astype(np.float32)
    for Xin, Gin, xf, gf in ((X, G, t_bf16(X).astype(np.float32), t_bf16(G).astype(np.float32)),
                             (Xf32, Gf32, Xf32, Gf32)):
        for eps in (1e-6, 0.25):
            Y = oracle.rmsnorm(Xin, Gin, eps)
            y_seq = _rmsnorm_fp32_sequential(xf, gf, eps).astype(np.float64)
            s_pw = np.sum(xf * xf, axis=-1, dtype=np.float32)
            r_pw = np.float32(1.0) / np.sqrt(s_pw / np.float32(D) + np.float32(eps), dtype=np.float32)
            y_pw = ((xf * r_pw[:, None]).astype(np.float32) * gf).astype(np.float64)
            t32, t16 = oracle.rmsnorm_tol(D, False), oracle.rmsnorm_tol(D, True)
            for y, t in ((y_seq, t32), (y_pw, t32), (_bf16_rne(y_seq), t16)):
                assert (np.abs(y - Y) <= t * np.abs(Y)).all(), (D, eps, float((np.abs(y - Y) / np.abs(Y)).max()), t)


def test_rmsnorm_tol_rejects_plausible_slips():
    """The same bound rejects a mean over D - 1 elements wherever it separates from it
    (D <= 2048: that slip moves every output by about 1/(2D) relative, the bound grows as
    D u / 2), a dropped eps and eps outside the root (eps = 0.25 against a mean square of
    about 0.25), and a truncated bf16 output. It says exactly where the D - 1 slip stops
    being separable, so that the GPU tests keep rows short enough to catch it."""
    from bigemm_inputs import normal_bf16
    from oracle_pins_lib import t_bf16
    separable = [D for D in (8, 64, 512, 1024, 2048, 4096, 8192) if 1.0 / (2 * D) > oracle.rmsnorm_tol(D, False)]
    assert separable == [8, 64, 512, 1024, 2048]
    for D in (8, 64, 520, 1024):
        X, G = normal_bf16(2410 + D, (4, D), 0.5), normal_bf16(2411, (D,))
        xf, gf = t_bf16(X).astype(np.float32), t_bf16(G).astype(np.float32)
        t32, t16 = oracle.rmsnorm_tol(D, False), oracle.rmsnorm_tol(D, True)
        Y = oracle.rmsnorm(X, G, 1e-6)
        slip = _rmsnorm_fp32_sequential(xf, gf, 1e-6, D=D - 1).astype(np.float64)
        assert (np.abs(slip - Y) > t32 * np.abs(Y)).any(), D
        Y25 = oracle.rmsnorm(X, G, 0.25)
        no_eps = _rmsnorm_fp32_sequential(xf, gf, 0.0).astype(np.float64)
        assert (np.abs(no_eps - Y25) > t16 * np.abs(Y25)).any(), D
        s = np.sum(xf * xf, axis=-1, dtype=np.float32) / np.float32(D)
        outside = (xf / (np.sqrt(s)[:, None] + np.float32(0.25)) * gf).astype(np.float64)
        assert (np.abs(outside - Y25) > t16 * np.abs(Y25)).any(), D
        y_ok = _rmsnorm_fp32_sequential(xf, gf, 1e-6)
        assert (np.abs(_bf16_trunc(y_ok) - Y) > t16 * np.abs(Y)).any(), D


@pytest.mark.parametrize("K", [64, 4096])
def test_parity_tol_bf16_out_admits_rne_and_rejects_slips(K):
    """PARITY_TOL_BF16_OUT (normalised by S = sum_k |x w|) admits a plain float32 GEMM of
    bf16 operands rounded once to bf16 (RNE), for a sequential and a library (BLAS) order,
    and rejects a truncated bf16 rounding, a row taken from the neighbouring input row and,
    at K = 64 where one product is 1/64 of S, a dropped last product. Positive operands make
    |y| = S, so the output rounding shows at full size."""
    from bigemm_inputs import f32_to_bf16_bits
    from oracle_pins_lib import t_bf16
    rng = np.random.default_rng(2420 + K)
    X = f32_to_bf16_bits(rng.uniform(0.5, 1.0, (48, K)).astype(np.float32))
    W = f32_to_bf16_bits(rng.uniform(0.5, 1.0, (K, 40)).astype(np.float32))
    Y, S = oracle.gemm_bf16(X, W)
    xf, wf = t_bf16(X).astype(np.float32), t_bf16(W).astype(np.float32)
    acc = np.zeros((48, 40), np.float32)
    for k in range(K):                       # float32, k ascending: one valid order
        acc += xf[:, k:k + 1] * wf[k:k + 1, :]
    tol = oracle.PARITY_TOL_BF16_OUT
    assert oracle.PARITY_TOL < tol < 2.0 ** -7
    assert oracle.max_normalized_error(_bf16_rne(acc), Y, S) <= tol
    assert oracle.max_normalized_error(_bf16_rne(xf @ wf), Y, S) <= tol
    assert oracle.max_normalized_error(_bf16_trunc(acc), Y, S) > tol
    assert oracle.max_normalized_error(_bf16_rne(np.roll(acc, 1, axis=0)), Y, S) > tol
    if K == 64:
        dropped = acc - xf[:, K - 1:K] * wf[K - 1:K, :]
        assert oracle.max_normalized_error(_bf16_rne(dropped), Y, S) > tol
