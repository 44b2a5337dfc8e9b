"""Batch-invariant paged attention on the GPU, through the C ABI.

What the blog's section on batch-invariant attention asks for, checked here:
* the KV cache is written before attention (bigemm_kv_cache_write), each row
  exactly where the page table puts it, and nothing else is touched;
* each token's output agrees with the oracle's fp64 causal attention within
  oracle.attention_tol;
* its bytes do not depend on the batch (T, the other tokens, the token's index),
  on which physical blocks hold the positions, on max_context, or on whether the
  earlier positions were cached by earlier calls — the section's examples: with
  block size 32, 80 cached tokens plus 48 new ones against 128 at once, and token
  1000 with 999 cached against all 1000 together.
"""
import numpy as np
import pytest
import torch

import harness as H
import invariant_gemm_deterministic_amd as bg
import oracle
from bigemm_inputs import block_table, kv_bf16, normal_bf16
from gpu_util import DEV, dev_bf16, require_gpu

pytestmark = pytest.mark.gpu

NAN16 = 0x7FC0  # bf16 quiet NaN: the fill of never-written cache rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bf(a) -> torch.Tensor:
    return dev_bf16(a).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor's bytes (bf16 as uint16, fp32 as uint32)."""
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy().view(np.uint32)


class Paged:
    """Keys/values of each sequence by position (host bf16 bits) and a paged copy on the GPU."""

    def __init__(self, seed, lens, Hkv, D, bs, spare=3, max_blocks=0, table_seed=None):
        self.lens = list(lens)
        self.maxlen = max(self.lens)
        self.Hkv, self.D, self.bs = Hkv, D, bs
        self.K, self.V = kv_bf16(seed, self.lens, Hkv, D)
        self.bt, self.nblocks = block_table(seed + 2 if table_seed is None else table_seed, self.lens, bs, spare,
                                            max_blocks)
        shape = (self.nblocks, Hkv, bs, D)
        self.kc = torch.full(shape, NAN16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        self.vc = torch.full(shape, NAN16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        self.bt_d = i32(self.bt)

    @property
    def capacity(self):
        return self.bt.shape[1] * self.bs

    def write(self, seqs, poss):
        seqs, poss = np.asarray(seqs, np.int32), np.asarray(poss, np.int32)
        bg.kv_cache_write(bf(self.K[seqs, poss]), bf(self.V[seqs, poss]), self.kc, self.vc, self.bt_d, i32(seqs),
                          i32(poss))

    def all_tokens(self):
        seqs = np.concatenate([np.full(L, s) for s, L in enumerate(self.lens)]).astype(np.int32)
        poss = np.concatenate([np.arange(L) for L in self.lens]).astype(np.int32)
        return seqs, poss

    def write_all(self):
        self.write(*self.all_tokens())
        return self

    def attend(self, Q, seqs, poss, **kw):
        o = bg.paged_attention(bf(Q), self.kc, self.vc, self.bt_d, i32(seqs), i32(poss), **kw)
        torch.cuda.synchronize()
        return o


def scale_of(D):
    return float(np.float32(1.0 / np.sqrt(D)))


def assert_parity(o, Q, P, seqs, poss, bf16_out=False):
    O, S, st = oracle.attention(Q, P.K, P.V, seqs, poss, scale_of(P.D))
    tol = oracle.attention_tol(st, (np.asarray(poss) + 1)[:, None], P.D, bf16_out)
    e = oracle.normalized_error(o.float().cpu().numpy(), O, S)
    bad = e > tol[..., None]
    assert not bad.any(), f"{int(bad.sum())} outputs beyond the bound; worst {float(e.max())} vs {float(tol.min())}"
    return float(e.max())


def sample_tokens(lens, extra=(0, 1, 255, 256, 257, 511, 512, 767)):
    seqs, poss = [], []
    for s, L in enumerate(lens):
        for p in sorted({q for q in extra if q < L} | {L - 1, L // 2}):
            seqs.append(s)
            poss.append(p)
    return np.array(seqs, np.int32), np.array(poss, np.int32)


# ------------------------------------------------------------------ KV-cache write
@pytest.mark.parametrize("bs", [1, 16, 32, 4096])
def test_kv_cache_write_places_rows(bs):
    P = Paged(300, [1, 31, 32, 33, 100], 2, 64, bs).write_all()
    want_k = np.full((P.nblocks, P.Hkv, bs, P.D), NAN16, np.uint16)
    want_v = want_k.copy()
    for s, L in enumerate(P.lens):
        j = np.arange(L)
        blk, row = P.bt[s, j // bs], j % bs
        want_k[blk, :, row] = P.K[s, :L]
        want_v[blk, :, row] = P.V[s, :L]
    assert np.array_equal(bits(P.kc), want_k)
    assert np.array_equal(bits(P.vc), want_v)


def test_kv_cache_write_skips_invalid_tokens():
    """Tokens whose sequence, position or block id is out of range write nothing."""
    P = Paged(310, [40, 10], 2, 128, 16)
    P.bt[1, 0] = P.nblocks + 7  # an invalid block id
    P.bt_d = i32(P.bt)
    before = (bits(P.kc).copy(), bits(P.vc).copy())
    kn, vn = bf(normal_bf16(311, (5, 2, 128))), bf(normal_bf16(312, (5, 2, 128)))
    bg.kv_cache_write(kn, vn, P.kc, P.vc, P.bt_d, i32([-1, 2, 0, 0, 1]), i32([0, 0, -1, P.capacity, 3]))
    torch.cuda.synchronize()
    assert np.array_equal(bits(P.kc), before[0]) and np.array_equal(bits(P.vc), before[1])


# ------------------------------------------------------------------ parity
PARITY = [  # (D, H, Hkv, bs, out_dtype)
    (128, 8, 8, 32, torch.float32),
    (128, 32, 8, 16, torch.float32),
    (64, 16, 2, 1, torch.float32),
    (64, 4, 2, 4096, torch.float32),
    (128, 16, 2, 64, torch.bfloat16),
    (64, 8, 2, 32, torch.bfloat16),
    (128, 32, 2, 32, torch.float32),
    (64, 16, 1, 16, torch.bfloat16),
    # group sizes that are not powers of two (28 query heads over 4 KV heads is a common layout)
    (128, 28, 4, 32, torch.float32),
    (64, 9, 3, 16, torch.bfloat16),
    (128, 10, 2, 8, torch.float32),
    (128, 12, 2, 64, torch.bfloat16),
    (64, 15, 1, 32, torch.float32),
]


@pytest.mark.parametrize("D,Hq,Hkv,bs,odt", PARITY)
def test_paged_attention_parity(D, Hq, Hkv, bs, odt):
    lens = [1, 256, 257, 700, 1030]
    P = Paged(320 + D + Hq, lens, Hkv, D, bs).write_all()
    seqs, poss = sample_tokens(lens)
    Q = normal_bf16(330 + Hq, (len(seqs), Hq, D))
    o = P.attend(Q, seqs, poss, out_dtype=odt)
    assert o.dtype == odt and tuple(o.shape) == (len(seqs), Hq, D)
    assert_parity(o, Q, P, seqs, poss, bf16_out=odt == torch.bfloat16)


def test_paged_attention_every_position_of_a_sequence():
    """All 600 positions of one sequence as queries (prefill shape) and a second sequence."""
    P = Paged(340, [600, 90], 4, 128, 32).write_all()
    seqs, poss = P.all_tokens()
    Q = normal_bf16(341, (len(seqs), 16, 128))
    assert_parity(P.attend(Q, seqs, poss), Q, P, seqs, poss)


def test_bf16_output_is_the_rounded_f32_output():
    from test_gpu_dtypes import rne_bf16_bits
    P = Paged(350, [300, 1200], 2, 128, 32).write_all()
    seqs, poss = sample_tokens(P.lens)
    Q = normal_bf16(351, (len(seqs), 8, 128))
    o32 = P.attend(Q, seqs, poss)
    obf = P.attend(Q, seqs, poss, out_dtype=torch.bfloat16)
    assert np.array_equal(bits(obf), rne_bf16_bits(o32.cpu().numpy()))


# ------------------------------------------------------------------ invariance
def test_batch_composition_and_index_do_not_matter():
    """Five target tokens alone (T = 1 each), inside two different batches of 64 tokens at
    different indices, and with a larger max_context: identical bytes."""
    lens = [600, 1, 300, 1300, 257, 40]
    P = Paged(360, lens, 4, 128, 32, max_blocks=200).write_all()
    Hq = 16
    tseq = np.array([3, 3, 0, 1, 4], np.int32)
    tpos = np.array([1299, 700, 599, 0, 256], np.int32)
    Qt = normal_bf16(361, (5, Hq, 128))
    alone = [P.attend(Qt[i:i + 1], tseq[i:i + 1], tpos[i:i + 1])[0] for i in range(5)]
    rng = np.random.default_rng(362)
    for trial, mc in enumerate([None, 1300, P.capacity]):
        fs = rng.integers(0, len(lens), 64).astype(np.int32)
        fp = np.array([rng.integers(0, lens[s]) for s in fs], np.int32)
        Qb = normal_bf16(363 + trial, (64, Hq, 128))
        idx = rng.choice(64, 5, replace=False)
        fs[idx], fp[idx], Qb[idx] = tseq, tpos, Qt
        ob = P.attend(Qb, fs, fp, max_context=mc)
        for i in range(5):
            assert H.byte_diff(ob[idx[i]], alone[i]) == 0, (trial, i)


def test_long_context_parity_and_max_context():
    """A 9000-position sequence (36 splits) against the oracle, and tokens of a
    300-position sequence computed in that call and again with max_context = 300 (a grid
    of 2 splits per token and a 2-split workspace stride): identical bytes."""
    P = Paged(365, [9000, 300], 2, 64, 32).write_all()
    seqs = np.array([0, 0, 0, 1, 1], np.int32)
    poss = np.array([8999, 4500, 256, 299, 40], np.int32)
    Q = normal_bf16(366, (5, 8, 64))
    o = P.attend(Q, seqs, poss, max_context=9000)
    assert_parity(o, Q, P, seqs, poss)
    short = P.attend(Q[3:], seqs[3:], poss[3:], max_context=300)
    assert H.byte_diff(o[3:], short) == 0


def test_physical_blocks_do_not_matter():
    P1 = Paged(370, [900, 77], 2, 64, 16).write_all()
    P2 = Paged(370, [900, 77], 2, 64, 16, spare=11, table_seed=999).write_all()
    assert not np.array_equal(P1.bt, P2.bt[:, :P1.bt.shape[1]])
    seqs, poss = P1.all_tokens()
    Q = normal_bf16(371, (len(seqs), 8, 64))
    assert H.byte_diff(P1.attend(Q, seqs, poss), P2.attend(Q, seqs, poss)) == 0


@pytest.mark.parametrize("L,first", [(128, 80), (1000, 999), (1000, 300)])
def test_cached_then_new_equals_all_at_once(L, first):
    """Block size 32. Whole: all L tokens written, then all L queried in one call. Chunked:
    tokens 0..first-1 written and queried, then the rest written and queried (the cache and
    table updated before attention each time). Every token's bytes agree."""
    Hq = 8
    Pw = Paged(380, [L], 2, 128, 32).write_all()
    seqs, poss = Pw.all_tokens()
    Q = normal_bf16(381, (L, Hq, 128))
    whole = Pw.attend(Q, seqs, poss)
    Pc = Paged(380, [L], 2, 128, 32)
    Pc.write(seqs[:first], poss[:first])
    a = Pc.attend(Q[:first], seqs[:first], poss[:first])
    Pc.write(seqs[first:], poss[first:])
    b = Pc.attend(Q[first:], seqs[first:], poss[first:])
    assert H.byte_diff(whole[:first], a) == 0
    assert H.byte_diff(whole[first:], b) == 0


def test_decode_token_by_token():
    """Ten decode steps, one token per step for each of three sequences: each step's outputs
    equal the outputs of the same tokens queried in one call after all writes."""
    lens = [270, 19, 520]
    P = Paged(390, lens, 2, 64, 32)
    seqs, poss = P.all_tokens()
    start = [L - 10 for L in lens]
    pre = np.concatenate([np.arange(start[s]) for s in range(3)])
    pre_s = np.concatenate([np.full(start[s], s) for s in range(3)])
    P.write(pre_s, pre)
    Q = normal_bf16(391, (3, 10, 8, 64))
    steps = []
    for k in range(10):
        ss = np.arange(3, dtype=np.int32)
        pp = np.array([start[s] + k for s in range(3)], np.int32)
        P.write(ss, pp)
        steps.append(P.attend(Q[:, k], ss, pp))
    allq = Q.transpose(1, 0, 2, 3).reshape(30, 8, 64)
    ss = np.tile(np.arange(3, dtype=np.int32), 10)
    pp = np.array([start[s] + k for k in range(10) for s in range(3)], np.int32)
    once = P.attend(allq, ss, pp)
    for k in range(10):
        assert H.byte_diff(steps[k], once[3 * k:3 * k + 3]) == 0, k


# ------------------------------------------------------------------ special cases
def test_nan_key_stays_in_its_sequence_and_heads():
    lens = [300, 300]
    Pn = Paged(400, lens, 2, 64, 32)
    Pn.K[0, 100, 0, 5] = NAN16
    Pn.write_all()
    Pc = Paged(400, lens, 2, 64, 32).write_all()
    seqs = np.array([0, 0, 0, 1, 1], np.int32)
    poss = np.array([99, 100, 299, 100, 299], np.int32)
    Q = normal_bf16(401, (5, 4, 64))
    on, oc = Pn.attend(Q, seqs, poss), Pc.attend(Q, seqs, poss)
    nan = torch.isnan(on)
    assert nan[1:3, :2].all() and not nan[1:3, 2:].any()  # heads 0,1 read KV head 0
    assert not nan[0].any() and not nan[3:].any()
    assert H.byte_diff(on[0], oc[0]) == 0 and H.byte_diff(on[3:], oc[3:]) == 0
    assert H.byte_diff(on[1:3, 2:], oc[1:3, 2:]) == 0


def test_invalid_tokens_and_blocks_give_nan_rows():
    P = Paged(410, [200, 200], 2, 64, 32)
    P.write_all()
    P.bt[1, 3] = -5  # positions 96..127 of sequence 1 now have no block
    P.bt_d = i32(P.bt)
    seqs = np.array([0, -1, 2, 0, 0, 1, 1], np.int32)
    poss = np.array([150, 10, 10, -1, 5000, 95, 96], np.int32)
    Q = normal_bf16(411, (7, 4, 64))
    o = P.attend(Q, seqs, poss, max_context=200)
    nan = torch.isnan(o).reshape(7, -1)
    assert nan[1:5].all() and nan[6].all()
    assert not nan[0].any() and not nan[5].any()
    ok = P.attend(Q[[0, 5]], seqs[[0, 5]], poss[[0, 5]])
    assert H.byte_diff(o[[0, 5]], ok) == 0


def test_bad_arguments_launch_nothing():
    P = Paged(420, [64], 2, 64, 32).write_all()
    kv = bg.bigemm_kv_layout(2, 64, 32, P.nblocks, 1, P.bt.shape[1])
    Q = bf(normal_bf16(421, (2, 4, 64)))
    seqs, poss = i32([0, 0]), i32([3, 63])
    out = torch.full((2, 4, 64), 7.0, device=DEV)
    need = bg.bigemm_attn_workspace_size(kv, 2, 4, 64)
    assert need == 2 * 4 * 1 * 66 * 4
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    args = (kv, 2, 4, 64, scale_of(64), bg.BIGEMM_F32, Q.data_ptr(), P.kc.data_ptr(), P.vc.data_ptr(),
            seqs.data_ptr(), poss.data_ptr(), P.bt_d.data_ptr(), out.data_ptr())
    assert bg.bigemm_paged_attention(*args, ws.data_ptr(), need - 4, 0, check=False) == bg.BIGEMM_ERR_ARG
    assert bg.bigemm_paged_attention(*args, ws.data_ptr() + 4, need, 0, check=False) == bg.BIGEMM_ERR_ARG
    bad = (kv, 2, 34, 64) + args[4:]  # 34 heads over 2 KV heads: a group of 17 is more than one MFMA tile
    assert bg.bigemm_paged_attention(*bad, ws.data_ptr(), 1 << 20, 0, check=False) == bg.BIGEMM_ERR_ARG
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    assert bg.bigemm_paged_attention(*args, ws.data_ptr(), need, 0, check=False) == bg.BIGEMM_OK
    torch.cuda.synchronize()
    assert not (out == 7.0).any()


# ------------------------------------------------------------------ full-size decode workload
def test_decode_workload_sampled():
    """The measured decode workload (64 sequences of 4096 positions, 32 query heads over 8
    KV heads of 128, block 32, one token per sequence at its last position): oracle parity
    on three sequences' tokens, and each of them alone gives the bytes of the full batch."""
    B, L, Hq, Hkv, D = 64, 4096, 32, 8, 128
    P = Paged(430, [L] * B, Hkv, D, 32).write_all()
    seqs = np.arange(B, dtype=np.int32)
    poss = np.full(B, L - 1, np.int32)
    Q = normal_bf16(431, (B, Hq, D))
    o = P.attend(Q, seqs, poss)
    pick = np.array([0, 31, 63])
    assert_parity(o[torch.as_tensor(pick)], Q[pick], P, seqs[pick], poss[pick])
    for i in pick:
        assert H.byte_diff(P.attend(Q[i:i + 1], seqs[i:i + 1], poss[i:i + 1])[0], o[i]) == 0, i


@pytest.mark.parametrize("D,out", [(128, "f32"), (128, "bf16"), (64, "f32"), (64, "bf16")])
def test_merge_thread_mappings_agree(D, out):
    """The merge spreads each output element over 32 threads when the call has few
    (token, head) pairs, and over 8 from 2048 workgroups of the narrow mapping on
    (T * H * D / 32 >= 2048: with 16 heads, from 32 tokens at D = 128 and from 64 at D = 64).
    Both mappings compute the same lane sums and tree, so the tokens just below the
    threshold (wide) and the same tokens inside a call at the threshold (narrow) give
    identical bytes, for each head dimension and output type (each pairing of compiled
    merge instances)."""
    lens = [3000, 700, 257]
    P = Paged(470 + D, lens, 4, D, 32).write_all()
    Hq = 16
    T = 2048 * 32 // (Hq * D)
    rng = np.random.default_rng(471 + D)
    seqs = rng.integers(0, len(lens), T).astype(np.int32)
    poss = np.array([rng.integers(0, lens[s]) for s in seqs], np.int32)
    Q = normal_bf16(472 + D, (T, Hq, D))
    odt = torch.float32 if out == "f32" else torch.bfloat16
    wide = P.attend(Q[:T - 1], seqs[:T - 1], poss[:T - 1], out_dtype=odt)
    narrow = P.attend(Q, seqs, poss, out_dtype=odt)
    assert H.byte_diff(narrow[:T - 1], wide) == 0
    if out == "f32":
        assert_parity(narrow, Q, P, seqs, poss)
    else:
        from test_gpu_dtypes import rne_bf16_bits
        n32 = P.attend(Q, seqs, poss)
        assert np.array_equal(bits(narrow), rne_bf16_bits(n32.cpu().numpy()))


@pytest.mark.parametrize("D", [64, 128])
def test_every_group_size(D):
    """Every group size G = H / Hkv from 1 to 16 has its own compiled split kernel: each
    against the oracle on tokens that end inside the first split, on a split boundary and in
    a later split (one KV head, so H = G)."""
    lens = [1, 257, 700]
    P = Paged(480 + D, lens, 1, D, 32).write_all()
    seqs = np.array([0, 1, 1, 2, 2], np.int32)
    poss = np.array([0, 0, 256, 255, 699], np.int32)
    for G in range(1, 17):
        Q = normal_bf16(481 + G, (len(seqs), G, D))
        o = P.attend(Q, seqs, poss)
        assert_parity(o, Q, P, seqs, poss)
