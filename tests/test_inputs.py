"""Seeded input generators: rounding, reproducibility and cell construction (CPU)."""
import numpy as np
import torch

import bigemm_inputs as G


def _torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_ties_and_torch_agreement():
    # ties to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1.015625
    b = G.f32_to_bf16_bits(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32))
    assert G.bf16_bits_to_f32(b).tolist() == [1.0, 1.015625]
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * np.float32(37.0)
    assert np.array_equal(G.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1.0, 0.01, 40.0)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(G.f32_to_e4m3_codes(x), ref)
    # saturation beyond the largest finite value (448)
    assert G.f32_to_e4m3_codes(np.array([1000.0, -1e6]))[0] == 0x7E
    assert G.f32_to_e4m3_codes(np.array([-1e6]))[0] == 0xFE


def test_integer_generators_are_exact():
    xb = G.int_bf16(3, (50, 40))
    assert np.all(G.bf16_bits_to_f32(xb) == np.round(G.bf16_bits_to_f32(xb)))
    xe = G.int_e4m3(4, (50, 40))
    v = torch.from_numpy(xe).view(torch.float8_e4m3fn).float().numpy()
    assert np.all(v == np.round(v)) and v.min() >= -8 and v.max() <= 8


def test_seeds_reproducible_and_independent():
    a = G.normal_bf16(G.SEED_A, (4, 64))
    assert np.array_equal(a, G.normal_bf16(G.SEED_A, (4, 64)))
    assert not np.array_equal(a, G.normal_bf16(G.SEED_B, (4, 64)))


def test_scales():
    assert np.all(G.e8m0_scales(0, (3, 4), "id") == 127)
    v = G.e8m0_scales(5, (200, 64), "var")
    assert v.min() >= 123 and v.max() <= 131 and len(np.unique(v)) == 9
    kx = G.e8m0_kvar_scales(6, 8, 5, k_axis=1)
    assert kx.shape == (5, 8) and np.all(kx == kx[0])
    kw = G.e8m0_kvar_scales(6, 8, 5, k_axis=0)
    assert kw.shape == (8, 5) and np.all(kw == kw[:, :1])


def test_linspace_row0_rounds_to_minus_1000():
    a = G.linspace_bf16(-1000.0, 1000.0, 2048 * 4096)[:4096]
    assert np.all(G.bf16_bits_to_f32(a) == -1000.0)
    b = G.linspace_bf16(-1000.0, 1000.0, 64, (8, 8))
    assert G.bf16_bits_to_f32(b)[0, 0] == -1000.0 and G.bf16_bits_to_f32(b)[-1, -1] == 1000.0


def test_row_positions_and_ab_rows():
    assert G.row_positions(1) == [0]
    assert G.row_positions(2) == [0, 1]
    assert G.row_positions(32) == [0, 16, 31]
    make = lambda seed, n: G.normal_bf16(seed, (n, 16))
    XA, XB, C = G.ab_cell_rows(make, 8, 4)
    assert np.array_equal(XA[4], C[0]) and np.array_equal(XB[4], C[0])
    others = [i for i in range(8) if i != 4]
    assert not np.array_equal(XA[others], XB[others])


def test_kv_generator_is_seeded_per_sequence():
    """Each sequence's keys/values come from its own stream: the same for any set of
    other sequences, different across sequences, zero past the sequence's length."""
    K1, V1 = G.kv_bf16(5, [10, 20, 3], 2, 16)
    K2, V2 = G.kv_bf16(5, [10, 4], 2, 16, threads=1)
    assert np.array_equal(K1[0, :10], K2[0, :10]) and np.array_equal(V1[0, :10], V2[0, :10])
    assert not np.array_equal(K1[0, :3], K1[2, :3])
    assert not K1[2, 3:].any() and not V1[0, 10:].any()
    k, v = G.seq_kv_bf16(5, 1, 20, 2, 16)
    assert np.array_equal(k, K1[1]) and np.array_equal(v, V1[1])


def test_block_table_assigns_distinct_blocks():
    lens, bs = [1, 31, 32, 33, 100, 0], 16
    bt, nb = G.block_table(9, lens, bs, spare=5)
    need = [-(-L // bs) for L in lens]
    assert nb == sum(need) + 5 and bt.shape == (len(lens), max(need))
    used = np.concatenate([bt[s, :n] for s, n in enumerate(need)])
    assert len(set(used.tolist())) == len(used) and used.min() >= 0 and used.max() < nb
    for s, n in enumerate(need):
        assert (bt[s, n:] == -1).all()
    bt2, _ = G.block_table(9, lens, bs, spare=5)
    assert np.array_equal(bt, bt2)
    wide, _ = G.block_table(9, lens, bs, max_blocks=20)
    assert wide.shape == (len(lens), 20)
