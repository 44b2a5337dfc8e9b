"""Seeded synthetic inputs for the batch-invariant GEMM.

This module is shared by the CPU oracle and by the GPU path's tests and bench.
It only *produces* operand bytes (bf16 bits, OCP E4M3FN codes, E8M0 scale
bytes) and assembles the invariance cells; it holds none of the GEMM's
arithmetic (no decoding, no scaling, no products, no sums).

Workloads follow the three pages on batch invariance:

* normal operands, N(0, sigma), as in the Variant A/B contract of the CANN
  ops-transformer issue (section "test methodology");
* the linspace experiment of the nondeterminism blog (section "batch
  invariance": a = linspace(-1000, 1000, B*D) reshaped [B, D],
  b = linspace(-1000, 1000, D*D) reshaped [D, D]);
* MXFP8 operands with identity ("ID") or K-varying ("VAR") block scales, the
  scale combinations of the issue's parameter grid.

Seeds: every array comes from ``numpy.random.default_rng(seed)``; the seed
constants below name the role of each draw so the A and B variants of a cell
differ only in the rows that the contract lets differ.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SEED_W", "SEED_C", "SEED_A", "SEED_B", "SEED_X", "SCALE_SEED_OFFSET",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bf16", "int_bf16", "linspace_bf16",
    "f32_to_e4m3_codes", "normal_e4m3", "int_e4m3", "e8m0_scales", "e8m0_kvar_scales",
    "row_positions", "ab_cell_rows", "position_cell_rows", "block_table", "seq_kv_bf16", "kv_bf16",
]

# Seed roles (the pages give none; these are fixed here once).
SEED_W = 0       # shared weight W
SEED_C = 1       # content C of the target row
SEED_A = 2       # the other rows in variant A
SEED_B = 3       # the other rows in variant B
SEED_X = 4       # a full batch X for M sweeps
SCALE_SEED_OFFSET = 100  # MX scale draws use element seed + 100


# --------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even; returns uint16 bits.

    NaN stays NaN (quiet). The inputs built here are always finite.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).reshape(-1)
    r = np.empty(u.shape, np.uint16)
    # uint32 arithmetic in chunks: for every non-NaN pattern u + 0x8000 < 2^32
    step = 1 << 22
    for i in range(0, u.size, step):
        v = u[i:i + step]
        r[i:i + step] = ((v + (np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    nan = np.isnan(a).reshape(-1)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)).astype(np.uint16) | np.uint16(0x0040))
    return r.reshape(a.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bits to float32 (exact). Used by tests to build torch/numpy views."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma) drawn in float32 from ``default_rng(seed)``, scaled in float32, RNE to bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f32_to_bf16_bits(x)


def int_bf16(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 bits (exactly representable for |v| <= 256)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def normal_f16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma) drawn in float32 from ``default_rng(seed)``, rounded to IEEE binary16
    (numpy's float32 -> float16 conversion, round to nearest even); returned as uint16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return x.astype(np.float16).view(np.uint16)


def int_f16(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] as binary16 bits (exact for |v| <= 2048)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16).view(np.uint16)


def int_i8(seed: int, shape, lo: int = -128, hi: int = 127) -> np.ndarray:
    """Uniform int8 values in [lo, hi] (the full range by default)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.int8)


def linspace_bf16(lo: float, hi: float, n: int, shape=None) -> np.ndarray:
    """The blog's linspace operand, rounded to bf16 in two explicit steps.

    v_i = lo + (hi - lo) * i / (n - 1) evaluated in float64, then RNE to
    float32, then RNE to bf16.
    """
    i = np.arange(n, dtype=np.float64)
    v = lo + ((hi - lo) * i) / float(n - 1)
    out = f32_to_bf16_bits(v.astype(np.float32))
    return out.reshape(shape) if shape is not None else out


# --------------------------------------------------------------------------- MXFP8
_E4M3_MAX = 448.0


def f32_to_e4m3_codes(a) -> np.ndarray:
    """Encode values as OCP E4M3FN codes (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, no infinities), round-to-nearest-even, saturating at +-448.

    Subnormals are m/8 * 2^-6 (exponent field 0). The input is finite.
    """
    x = np.asarray(a, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    mag = np.minimum(np.abs(x), _E4M3_MAX)
    # binade exponent (exact via frexp), floored at the subnormal exponent -6
    e = np.frexp(np.where(mag > 0, mag, 1.0))[1].astype(np.float64) - 1.0
    e = np.clip(e, -6, 8)
    q = np.exp2(e - 3)                      # spacing of representable values in this binade
    r = np.rint(mag / q) * q                # RNE onto the grid (exact scaling by powers of 2)
    r = np.minimum(r, _E4M3_MAX)
    # re-derive exponent after rounding (a carry can move r to the next binade)
    e2 = np.frexp(np.where(r > 0, r, 1.0))[1].astype(np.float64) - 1.0
    sub = r < 2.0 ** -6
    m_sub = np.rint(r / 2.0 ** -9)
    m_nrm = np.rint(r / np.exp2(e2 - 3)) - 8
    code = np.where(sub, m_sub, (e2 + 7) * 8 + m_nrm)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def normal_e4m3(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma) drawn in float32, RNE to E4M3FN (saturation never reached in practice)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f32_to_e4m3_codes(x)


def int_e4m3(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] as E4M3FN codes (exact for |v| <= 16)."""
    rng = np.random.default_rng(seed)
    return f32_to_e4m3_codes(rng.integers(lo, hi + 1, size=shape).astype(np.float64))


def e8m0_scales(seed: int, shape, kind: str = "id", lo: int = -4, hi: int = 4) -> np.ndarray:
    """E8M0 block-scale bytes. ``id``: every byte 127 (2^0). ``var``: independent
    uniform exponents in [lo, hi], byte = 127 + exponent.

    ``shape`` is (rows, K/32) for X scales and (K/32, cols) for W scales.
    """
    if kind == "id":
        return np.full(shape, 127, dtype=np.uint8)
    rng = np.random.default_rng(seed)
    if kind == "var":
        return (127 + rng.integers(lo, hi + 1, size=shape)).astype(np.uint8)
    raise ValueError(f"unknown scale kind {kind!r}")


def e8m0_kvar_scales(seed: int, n_kblocks: int, n_other: int, k_axis: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Scales that vary along K only (one exponent per K block, same for every row or column)."""
    rng = np.random.default_rng(seed)
    v = (127 + rng.integers(lo, hi + 1, size=n_kblocks)).astype(np.uint8)
    if k_axis == 1:   # X scales [rows, K/32]
        return np.tile(v[None, :], (n_other, 1))
    return np.tile(v[:, None], (1, n_other))


# --------------------------------------------------------------------------- cells
def row_positions(M: int):
    """Target rows of a cell: 0, mid = floor(M/2), last = M-1 (deduplicated, ordered)."""
    out = []
    for r in (0, M // 2, M - 1):
        if r not in out:
            out.append(r)
    return out


def ab_cell_rows(make_rows, M: int, row: int, seed_C: int = SEED_C, seed_A: int = SEED_A, seed_B: int = SEED_B):
    """Variant A and B batches for one cell of the A/B contract.

    ``make_rows(seed, n)`` returns n rows (a 2-D array). Both variants hold
    the same content C at ``row``; the other rows come from seed_A or seed_B.
    Returns (X_A, X_B, C) with C of shape [1, ...].
    """
    C = make_rows(seed_C, 1)
    XA = make_rows(seed_A, M).copy()
    XB = make_rows(seed_B, M).copy()
    XA[row] = C[0]
    XB[row] = C[0]
    return XA, XB, C


def position_cell_rows(make_rows, M: int, row: int, seed_C: int = SEED_C, seed_fill: int = SEED_A):
    """One batch with content C placed at ``row`` and seeded filler elsewhere."""
    C = make_rows(seed_C, 1)
    X = make_rows(seed_fill, M).copy()
    X[row] = C[0]
    return X, C


# ------------------------------------------------------------------ paged KV cache
def block_table(seed: int, lens, block_size: int, spare: int = 0, max_blocks: int = 0):
    """A page table for sequences of lengths ``lens``: sequence s owns ceil(lens[s] /
    block_size) physical blocks, drawn without repetition from a shuffled pool of all the
    blocks needed plus ``spare`` unused ones. Returns (table [len(lens), max_blocks] int32,
    padded with -1, and the pool size num_blocks). Layout only: no attention arithmetic."""
    need = [-(-int(L) // block_size) for L in lens]
    num_blocks = sum(need) + spare
    pool = np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)
    width = max(max(need), max_blocks, 1)
    table = np.full((len(lens), width), -1, np.int32)
    off = 0
    for s, n in enumerate(need):
        table[s, :n] = pool[off:off + n]
        off += n
    return table, num_blocks


def seq_kv_bf16(seed: int, s: int, L: int, Hkv: int, D: int):
    """Keys and values of sequence s, N(0, 1) rounded to bf16, each [L, Hkv, D], drawn in
    float32 from default_rng((seed, s)) — one stream per sequence, so sequences can be
    made independently and in parallel."""
    x = np.random.default_rng((seed, s)).standard_normal((2, L, Hkv, D), dtype=np.float32)
    b = f32_to_bf16_bits(x)
    return b[0], b[1]


def kv_bf16(seed: int, lens, Hkv: int, D: int, threads: int = 8):
    """Keys and values of every sequence, [len(lens), max(lens), Hkv, D] each (positions
    past a sequence's length are zero), from seq_kv_bf16."""
    from concurrent.futures import ThreadPoolExecutor

    lens = [int(L) for L in lens]
    K = np.zeros((len(lens), max(lens), Hkv, D), np.uint16)
    V = np.zeros_like(K)

    def fill(s):
        K[s, :lens[s]], V[s, :lens[s]] = seq_kv_bf16(seed, s, lens[s], Hkv, D)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(len(lens))))
    return K, V
