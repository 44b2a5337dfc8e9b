"""The invariance harness passes batch-invariant GEMMs and catches each planted
batch dependence (CPU only)."""
import json
import os

import numpy as np
import pytest

import harness as H
import negative_controls as NC
from bigemm_inputs import SEED_W, SEED_X, normal_bf16, normal_e4m3, e8m0_scales, row_positions


def _mboundaries(golden_dir):
    with open(os.path.join(golden_dir, "m_boundaries.txt")) as f:
        return [int(v) for ln in f if not ln.startswith("#") for v in ln.split()]


@pytest.fixture(scope="module")
def cfg1_weights():
    # X[M,256] . W[256,128], N(0,1) (the small bf16 workload)
    return (normal_bf16(SEED_W, (256, 128)),)


@pytest.mark.parametrize("gemm", [NC.gemm_oracle, NC.gemm_ordered_f32], ids=["oracle", "ordered_f32"])
def test_harness_passes_invariant_gemm(gemm, cfg1_weights):
    make = H.rows_bf16(256)
    for M in (1, 4, 8, 16, 32):
        for r in row_positions(M):
            cell = H.ab_cell(gemm, make, cfg1_weights, M, r)
            assert cell["ab"] == 0 and cell["canon"] == 0, cell
        assert all(v == 0 for v in H.position_cell(gemm, make, cfg1_weights, M).values())
    X = make(SEED_X, 32)
    assert H.repeat_cell(gemm, X, cfg1_weights) == 0


def test_harness_passes_oracle_msweep(golden_dir):
    K, N = 512, 32
    W = (normal_bf16(SEED_W, (K, N), 0.02),)
    X = (normal_bf16(SEED_X, (256, K)),)
    out = H.msweep_cell(NC.gemm_oracle, X, W, _mboundaries(golden_dir))
    assert all(v["rows"] == 0 and v["alone"] == 0 for v in out.values()), out


def test_nc1_msplit_caught_by_msweep(golden_dir):
    """Projection magnitudes (X ~ N(0,1), W ~ N(0,0.02)): the M sweep must see byte
    diffs at the 64-row boundaries of the split-count formula."""
    K, N = 1024, 32
    W = (normal_bf16(SEED_W, (K, N), 0.02),)
    X = (normal_bf16(SEED_X, (256, K)),)
    out = H.msweep_cell(NC.gemm_nc1_msplit, X, W, _mboundaries(golden_dir))
    changed = [M for M, v in out.items() if v["rows"] > 0]
    assert changed, out
    # rows of batches on the same side of every boundary as the full batch agree
    assert out[256]["rows"] == 0 and out[193]["rows"] == 0
    # and each crossing of a 64-row boundary is seen
    assert {1, 64, 65, 128, 129, 192}.issubset(changed)


def test_nc2_amax_caught_by_ab_cell(cfg1_weights):
    make = H.rows_bf16(256)
    diffs = [H.ab_cell(NC.gemm_nc2_amax, make, cfg1_weights, M, r)["ab"]
             for M in (4, 8, 16, 32) for r in row_positions(M)]
    assert all(d > 0 for d in diffs), diffs


def test_nc3_position_caught_by_position_cell(cfg1_weights):
    make = H.rows_bf16(256)
    d = H.position_cell(NC.gemm_nc3_position, make, cfg1_weights, 32)
    assert d[0] == 0 and d[16] > 0 and d[31] > 0, d


def test_nc2_caught_on_mxfp8():
    """The content-dependent control also fails on MXFP8 operands with VAR scales."""
    K, N = 256, 64
    Wt = (normal_e4m3(SEED_W, (K, N)), e8m0_scales(SEED_W + 100, (K // 32, N), "var"))
    make = H.rows_mx(K, "var")
    assert H.ab_cell(NC.gemm_nc2_amax, make, Wt, 16, 8)["ab"] > 0
    assert H.ab_cell(NC.gemm_oracle, make, Wt, 16, 8)["ab"] == 0


def test_byte_diff_counts_signed_zero_and_nan():
    a = np.array([0.0, 1.0, np.nan], dtype=np.float32)
    b = np.array([-0.0, 1.0, np.nan], dtype=np.float32)
    assert H.byte_diff(a, b) == 1          # +0 and -0 differ in the sign byte
    assert H.byte_diff(a, a.copy()) == 0   # identical NaN payloads are equal bytes


def test_cell_grid_fixture(golden_dir):
    with open(os.path.join(golden_dir, "bi_cell_grid.json")) as f:
        g = json.load(f)
    n = len(g["M_per_rank"]) * len(g["K"]) * len(g["N"]) * len(g["row_positions"]) * len(g["scale_combos"])
    assert n == 1440
    assert g["bi_standard"] == {"row_positions": [0, "mid", "last"], "n_variants": 2}
