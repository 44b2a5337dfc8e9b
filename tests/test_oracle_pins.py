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
