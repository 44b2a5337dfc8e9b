"""The oracle pinned to facts outside itself (see oracle_pins_lib for the sources)."""
import pytest

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
    import numpy as np
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
    import numpy as np
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
