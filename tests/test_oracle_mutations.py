"""Plant plausible mistakes in copies of the oracle's C source and check that the
pins catch every one of them (no GPU involved; the shipped oracle is untouched)."""
import os
import tempfile

import pytest

import oracle
import oracle_pins_lib as pins

# (name, text in oracle.c, replacement). Every replacement keeps memory accesses in bounds.
MUTATIONS = [
    ("drop_last_k", "for (int64_t k = 0; k < K; ++k) {\n      const double a = A[i * lda + k];",
     "for (int64_t k = 0; k < K - 1; ++k) {\n      const double a = A[i * lda + k];"),
    ("reverse_k_order", "for (int64_t k = 0; k < K; ++k) {\n      const double a = A[i * lda + k];",
     "for (int64_t k = K - 1; k >= 0; --k) {\n      const double a = A[i * lda + k];"),
    ("wrong_sign", "acc[j] += a * brow[j];", "acc[j] -= a * brow[j];"),
    ("row_index", "const double a = A[i * lda + k];", "const double a = A[(i > 0 ? i - 1 : 0) * lda + k];"),
    ("w_rows_reversed", "B[k * N + j] = oracle_decode_bf16(W[k * ldw + j]);",
     "B[k * N + j] = oracle_decode_bf16(W[(K - 1 - k) * ldw + j]);"),
    ("s_without_abs", "sabs[j] += fabs(a * brow[j]);", "sabs[j] += a * brow[j];"),
    ("bf16_low_bit", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)(bits & 0xFFFE) << 16;"),
    ("e4m3_bias", "v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    ("e4m3_subnormal", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3_nan", "if (e == 15 && m == 7) return NAN;", "if (e == 15 && m == 7) return 480.0;"),
    ("e8m0_bias", "return ldexp(1.0, (int)code - 127);", "return ldexp(1.0, (int)code - 126);"),
    ("x_scale_block", "oracle_decode_e8m0(XS[i * ldxs + k / 32])", "oracle_decode_e8m0(XS[i * ldxs + (k % 32) % ldxs])"),
    ("w_scale_column", "oracle_decode_e8m0(WS[(k / 32) * ldws + j])", "oracle_decode_e8m0(WS[(k / 32) * ldws + (N - 1 - j)])"),
    ("f16_bias", "v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    ("f16_subnormal", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -23);"),
    ("f16_inf", "if (e == 31) v = m ? NAN : INFINITY;", "if (e == 31) v = m ? NAN : 65536.0;"),
    ("i8_unsigned", "const int64_t a = X[i * ldx + k];", "const int64_t a = (uint8_t)X[i * ldx + k];"),
    ("i8_w_columns", "acc[j] += a * (int64_t)wrow[j];", "acc[j] += a * (int64_t)wrow[N - 1 - j];"),
    ("i8_drop_last_k", "for (int64_t k = 0; k < K; ++k) {\n      const int64_t a",
     "for (int64_t k = 0; k < K - 1; ++k) {\n      const int64_t a"),
    ("rms_not_squared", "for (int64_t j = 0; j < D; ++j) s += x[j] * x[j];", "for (int64_t j = 0; j < D; ++j) s += fabs(x[j]);"),
    ("rms_drop_last", "for (int64_t j = 0; j < D; ++j) s += x[j] * x[j];", "for (int64_t j = 0; j < D - 1; ++j) s += x[j] * x[j];"),
    ("rms_mean_d_minus_1", "sqrt(s / (double)D + eps)", "sqrt(s / (double)(D > 1 ? D - 1 : 1) + eps)"),
    ("rms_no_eps", "sqrt(s / (double)D + eps)", "sqrt(s / (double)D)"),
    ("rms_gamma_reversed", "Y[i * ldy + j] = x[j] / den * G[j];", "Y[i * ldy + j] = x[j] / den * G[D - 1 - j];"),
    ("rms_gamma_ignored", "for (int64_t j = 0; j < D; ++j) G[j] = oracle_decode_bf16(gamma[j]);",
     "for (int64_t j = 0; j < D; ++j) G[j] = 1.0;"),
    ("x_scale_dropped", "A[i * K + k] = e4m3_table[X[i * ldx + k]] * oracle_decode_e8m0(XS[i * ldxs + k / 32]);",
     "A[i * K + k] = e4m3_table[X[i * ldx + k]];"),
    ("attn_causal_exclusive", "const int64_t L = p + 1; /* keys j = 0 .. p */", "const int64_t L = p;"),
    ("attn_no_scale", "s[j] = scale * d;", "s[j] = d;"),
    ("attn_gqa_modulo", "const int64_t g = h / (H / Hkv);", "const int64_t g = h % Hkv;"),
    ("attn_no_max_shift", "w[j] = exp(s[j] - m);", "w[j] = exp(s[j]);"),
    ("attn_unnormalised", "O[(t * H + h) * D + e] = num / den;", "O[(t * H + h) * D + e] = num;"),
    ("attn_v_next_position", "V[((sq * maxlen + j) * Hkv + g) * D + e]",
     "V[((sq * maxlen + (j + 1 < L ? j + 1 : j)) * Hkv + g) * D + e]"),
    ("attn_seq_ignored", "const int64_t sq = seq[t];", "const int64_t sq = 0;"),
    ("attn_k_reversed", "q[e] * oracle_decode_bf16(k[e])", "q[e] * oracle_decode_bf16(k[D - 1 - e])"),
    ("attn_q_first_head_of_group", "Q[(t * H + h) * D + e]", "Q[(t * H + g * (H / Hkv)) * D + e]"),
    ("attn_s_signed", "nabs += w[j] * fabs(v);", "nabs += w[j] * v;"),
    ("attn_a_signed", "da += fabs(prod);", "da += prod;"),
    ("attn_range_from_zero", "stats[(t * H + h) * 3 + 2] = m - s_min;", "stats[(t * H + h) * 3 + 2] = m;"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(source, name, old, new):
    assert source.count(old) == 1, f"mutation {name} does not apply"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "oracle_mut.c")
        with open(src, "w") as f:
            f.write(source.replace(old, new))
        lib = oracle.build(force=True, src=src, out=os.path.join(d, "liboracle_mut.so"))
        orc = oracle.Oracle(lib)
        failed = []
        for check in pins.ALL_CHECKS:  # the first pin that fails is enough
            try:
                check(orc)
            except AssertionError:
                failed.append(check.__name__)
                break
        assert failed, f"no pin caught mutation {name}"
