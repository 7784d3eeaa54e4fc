"""Pins of the CPU oracle against facts it does not produce itself.

Each check is a function of the oracle routine it checks, so the mutation
tests at the bottom can hand it a routine with a planted mistake (on the CPU)
and see the check fail.

* unsplit attention: brute force at 50 digits (mpmath, scalar loops) and the
  closed forms of the softmax (identical keys, one token, constant V, two
  tokens, a dominant token);
* combine / split: the combine of any partition of the tokens (empty parts
  included) equals the unsplit result (the exactness claim of the review's
  Prompt 1.3.2);
* placement: the two-slice example of the NVIDIA blog's KV-placement section,
  a bijection check by enumeration, and the slice-length formula against
  enumeration;
* codecs: the OCP fp8 E4M3 / MX FP4 / E8M0 published values and torch's own
  float8_e4m3fn cast.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import attention, codecs, placement

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- attention

def brute_force_attention(q, K, V, scale, dps=50):
    """The definition evaluated term by term at ``dps`` digits."""
    with mpmath.workdps(dps):
        G, D = len(q), len(q[0])
        n, Dv = len(K), len(V[0])
        outs, lses = [], []
        for h in range(G):
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[h][d]) * mpmath.mpf(K[t][d]) for d in range(D))
                 for t in range(n)]
            z = mpmath.fsum(mpmath.exp(x) for x in s)
            lses.append(mpmath.log(z))
            outs.append([mpmath.fsum(mpmath.exp(s[t]) * mpmath.mpf(V[t][e]) for t in range(n)) / z
                         for e in range(Dv)])
        return (np.array([[float(x) for x in row] for row in outs]), np.array([float(x) for x in lses]))


def check_bruteforce(attend_fn):
    rng = np.random.default_rng(1234)
    for n, D, Dv, G, sd in [(1, 4, 3, 2, 1.0), (7, 8, 8, 3, 1.0), (64, 8, 5, 4, 2.0), (33, 5, 8, 1, 3.0)]:
        q = rng.normal(0, sd, (G, D))
        K = rng.normal(0, sd, (n, D))
        V = rng.normal(0, 1, (n, Dv))
        scale = 1.0 / math.sqrt(D)
        O, L = attend_fn(q, K, V, scale)
        Ob, Lb = brute_force_attention(q.tolist(), K.tolist(), V.tolist(), scale)
        assert np.max(np.abs(O - Ob)) <= 1e-13, (n, D, np.max(np.abs(O - Ob)))
        assert np.max(np.abs(L - Lb)) <= 1e-13 * max(1.0, np.max(np.abs(Lb))), (n, D)


def check_closed_forms(attend_fn):
    rng = np.random.default_rng(7)
    D, Dv, G = 16, 12, 3
    q = rng.normal(0, 1, (G, D))
    scale = 0.25
    # identical keys: uniform weights -> mean of V, LSE = s + ln n
    n = 37
    k = rng.normal(0, 1, D)
    K = np.tile(k, (n, 1))
    V = rng.normal(0, 1, (n, Dv))
    O, L = attend_fn(q, K, V, scale)
    s = scale * (q @ k)
    assert np.max(np.abs(O - V.mean(axis=0))) <= 1e-14
    assert np.max(np.abs(L - (s + math.log(n)))) <= 1e-13
    # one token: O = v, LSE = s
    O, L = attend_fn(q, K[:1], V[:1], scale)
    assert np.max(np.abs(O - V[0])) <= 1e-15 and np.max(np.abs(L - s)) <= 1e-14
    # constant V: O = c whatever the scores
    K = rng.normal(0, 2, (n, D))
    c = rng.normal(0, 1, Dv)
    O, _ = attend_fn(q, K, np.tile(c, (n, 1)), scale)
    assert np.max(np.abs(O - c)) <= 1e-14
    # two tokens: logistic weights
    K2 = rng.normal(0, 1, (2, D))
    V2 = rng.normal(0, 1, (2, Dv))
    O, L = attend_fn(q, K2, V2, scale)
    s1, s2 = scale * (q @ K2[0]), scale * (q @ K2[1])
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    w2 = 1.0 / (1.0 + np.exp(s1 - s2))
    assert np.max(np.abs(O - (w1[:, None] * V2[0] + w2[:, None] * V2[1]))) <= 1e-14
    assert np.max(np.abs(L - (np.maximum(s1, s2) + np.log1p(np.exp(-np.abs(s1 - s2)))))) <= 1e-13
    # a score gap above 800: exactly one-hot in fp64
    q1 = np.zeros((1, D))
    q1[0, 0] = 1.0
    Kd = np.zeros((5, D))
    Kd[3, 0] = 1000.0
    Vd = rng.normal(0, 1, (5, Dv))
    O, L = attend_fn(q1, Kd, Vd, 1.0)
    assert np.array_equal(O[0], Vd[3]) and L[0] == 1000.0


def test_attend_bruteforce():
    check_bruteforce(attention.attend)


def test_attend_closed_forms():
    check_closed_forms(attention.attend)


def test_attend_empty():
    O, L = attention.attend(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 3)), 1.0)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_attend_heads_grouping():
    rng = np.random.default_rng(3)
    Hq, Hkv, n, D = 6, 2, 20, 8
    q = rng.normal(size=(Hq, D))
    K = rng.normal(size=(Hkv, n, D))
    V = rng.normal(size=(Hkv, n, D))
    O, L = attention.attend_heads(q, K, V, 0.3)
    for h in range(Hq):
        Oh, Lh = attention.attend(q[h:h + 1], K[h // 3], V[h // 3], 0.3)
        assert np.max(np.abs(O[h] - Oh[0])) <= 1e-14 and abs(L[h] - Lh[0]) <= 1e-14


# ---------------------------------------------------------------- combine

def check_split_invariance(attend_fn, combine_fn, seed, n, parts):
    rng = np.random.default_rng(seed)
    G, D, Dv = 3, 8, 6
    q = rng.normal(0, 1.5, (G, D))
    K = rng.normal(0, 1.5, (n, D))
    V = rng.normal(0, 1, (n, Dv))
    scale = 1 / math.sqrt(D)
    O, L = attend_fn(q, K, V, scale)
    label = rng.integers(0, parts, n)
    Op = np.empty((parts, G, Dv))
    Lp = np.empty((parts, G))
    for p in range(parts):
        idx = np.nonzero(label == p)[0]
        Op[p], Lp[p] = attend_fn(q, K[idx], V[idx], scale)
    Oc, Lc = combine_fn(Op, Lp)
    assert np.max(np.abs(Oc - O)) <= 1e-12, np.max(np.abs(Oc - O))
    assert np.max(np.abs(Lc - L)) <= 1e-12 * max(1, np.max(np.abs(L)))


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n=st.integers(1, 300), parts=st.integers(1, 12))
def test_combine_any_partition(seed, n, parts):
    check_split_invariance(attention.attend, attention.combine, seed, n, parts)


def test_combine_all_empty():
    O, L = attention.combine(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_combine_single_part_is_identity():
    rng = np.random.default_rng(0)
    Op = rng.normal(size=(1, 4, 5))
    Lp = rng.normal(size=(1, 4))
    O, L = attention.combine(Op, Lp)
    assert np.array_equal(O, Op[0]) and np.array_equal(L, Lp[0])


@pytest.mark.parametrize("n,P", [(1, 4), (15, 4), (16, 4), (17, 4), (4096, 4), (1000, 8), (4137, 8), (33, 1)])
def test_round_robin_slices_combine_to_unsplit(n, P):
    rng = np.random.default_rng(n + P)
    q = rng.normal(size=(4, 16))
    K = rng.normal(size=(n, 16))
    V = rng.normal(size=(n, 16))
    O, L = attention.attend(q, K, V, 0.25)
    Op, Lp = attention.slice_partials(q, K, V, 0.25, P)
    Oc, Lc = attention.combine(Op, Lp)
    assert np.max(np.abs(Oc - O)) <= 1e-12 and np.max(np.abs(Lc - L)) <= 1e-12


def check_slice_partials(partials_fn):
    """Slice r's partial is the unsplit attention over exactly the tokens the
    placement enumerates for slice r (a slipped slice index or a wrong mask
    fails here even though the combine of all slices would not notice)."""
    rng = np.random.default_rng(99)
    for n, P in [(1, 3), (17, 2), (100, 3), (257, 4), (600, 8), (40, 8)]:
        q = rng.normal(size=(3, 8))
        K = rng.normal(size=(n, 8))
        V = rng.normal(size=(n, 6))
        Op, Lp = partials_fn(q, K, V, 0.3, P)
        for r in range(P):
            toks = placement.slice_tokens(n, P, r)
            O, L = attention.attend(q, K[toks], V[toks], 0.3)
            if not toks:
                assert np.all(Op[r] == 0) and np.all(np.isneginf(Lp[r])), (n, P, r)
                continue
            assert np.max(np.abs(Op[r] - O)) <= 1e-12, (n, P, r)
            assert np.max(np.abs(Lp[r] - L)) <= 1e-12 * max(1, np.max(np.abs(L))), (n, P, r)


def test_slice_partials_follow_the_placement():
    check_slice_partials(attention.slice_partials)


def test_slice_mask_matches_enumeration():
    for P in (1, 2, 3, 8):
        for n in (0, 1, 16, 17, 100, 257):
            for r in range(P):
                idx = np.nonzero(attention.slice_mask(n, P, r))[0].tolist()
                assert idx == placement.slice_tokens(n, P, r)


# ---------------------------------------------------------------- placement

def check_page_placement(slot_fn, golden):
    P = golden["P"]
    for lo, hi, rank in golden["ranges_1based_inclusive"]:
        for tok in range(lo, hi + 1):
            assert slot_fn(tok - 1, P)[0] == rank, (tok, rank)


def check_placement_bijection(slot_fn):
    for P in range(1, 9):
        for n in (1, 15, 16, 17, 31, 32, 33, 16 * P, 16 * P + 5, 333):
            seen = set()
            per_slice = {}
            for t in range(n):
                r, j = slot_fn(t, P)
                assert 0 <= r < P and j >= 0
                assert (r, j) not in seen
                seen.add((r, j))
                per_slice.setdefault(r, []).append((t, j))
            for r, rows in per_slice.items():
                js = [j for _, j in rows]
                assert js == list(range(len(js))), "rows of a slice are dense and in arrival order"
            lens = [len(per_slice.get(r, [])) for r in range(P)]
            assert max(lens) - min(lens) <= 16


def test_placement_page_example(golden_dir):
    with open(os.path.join(golden_dir, "placement_two_slices.json")) as f:
        check_page_placement(placement.slot, json.load(f))


def test_placement_bijection():
    check_placement_bijection(placement.slot)


def test_placement_16_token_rotation():
    # a new slice every 16 tokens, cycling through all P slices
    for P in (2, 4, 8):
        ranks = [placement.slot(t, P)[0] for t in range(16 * P * 3)]
        assert ranks == [(t // 16) % P for t in range(16 * P * 3)]


def test_slice_len_matches_enumeration():
    for P in range(1, 10):
        for n in list(range(0, 16 * P * 2 + 3)) + [4096, 4137, 131071]:
            if n > 5000 and P not in (4, 8):
                continue
            for r in range(P):
                assert placement.slice_len(n, P, r) == len(placement.slice_tokens(n, P, r)), (n, P, r)


def test_slice_len_examples():
    # 4137 tokens over 8 slices: 32 full rounds of 128, then 41 left = 16+16+9
    assert [placement.slice_len(4137, 8, r) for r in range(8)] == [528, 528, 521, 512, 512, 512, 512, 512]
    assert [placement.slice_len(4096, 4, r) for r in range(4)] == [1024] * 4
    assert placement.slice_len(1 << 20, 8, 5) == 131072


def test_blocks_needed_is_the_ceiling_of_the_slice_rows():
    for P in (1, 2, 3, 8):
        for n in list(range(0, 16 * P * 3 + 5)) + [4137]:
            for r in range(P):
                assert placement.blocks_needed(n, P, r) == -(-placement.slice_len(n, P, r) // 16), (n, P, r)


def test_block_rows_are_a_bijection_onto_the_listed_blocks():
    """Every token of a request lands on its own (block, row); the blocks in
    use are exactly the first blocks_needed entries of each slice's list;
    tokens of one 16-token group share a block in arrival order."""
    rng = np.random.default_rng(7)
    for P in (1, 2, 5, 8):
        for n in (1, 15, 16, 17, 16 * P, 16 * P + 1, 700, 4137):
            nb = [placement.blocks_needed(n, P, r) for r in range(P)]
            ids = rng.permutation(sum(nb) + 11)          # a pool with spare blocks, shuffled
            table, k = [], 0
            for r in range(P):
                table.append(list(ids[k:k + nb[r]]) + [-1] * 3)
                k += nb[r]
            where = [placement.block_row(t, P, table) for t in range(n)]
            assert len(set(where)) == n
            assert all(blk >= 0 and 0 <= row < 16 for blk, row in where)
            used = {blk for blk, _ in where}
            assert used == {table[r][c] for r in range(P) for c in range(nb[r])}
            for t in range(n):
                g0 = (t // 16) * 16
                assert where[t] == (where[g0][0], t - g0)


# ---------------------------------------------------------------- codecs

def _spec_value(v):
    return float("nan") if v == "nan" else float(v)


def check_codec_spec(fp8_table, e2m1_table, e8m0_table, golden):
    for code, v in golden["fp8_e4m3"].items():
        got = fp8_table[int(code)]
        want = _spec_value(v)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    for code, want in enumerate(golden["e2m1"]):
        assert e2m1_table[code] == want and math.copysign(1, e2m1_table[code]) == math.copysign(1, want), code
    for code, v in golden["e8m0"].items():
        want = _spec_value(v)
        got = e8m0_table[int(code)]
        assert (math.isnan(got) and math.isnan(want)) or got == want, code


def test_codecs_against_spec(golden_dir):
    with open(os.path.join(golden_dir, "ocp_formats.json")) as f:
        check_codec_spec(codecs.FP8_E4M3, codecs.E2M1, codecs.E8M0, json.load(f))


def test_fp8_table_matches_torch_cast():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.FP8_E4M3
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))


def test_fp8_table_monotone_and_max():
    pos = codecs.FP8_E4M3[:127]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0


def test_dequant_fp8_chunks():
    codes = np.array([[0x38] * 8] * 20, dtype=np.uint8)  # 1.0 everywhere, 20 tokens
    scales = np.array([0.5, 3.0], dtype=np.float32)
    out = codecs.dequant_fp8(codes, scales)
    assert np.all(out[:16] == 0.5) and np.all(out[16:] == 3.0)
    # the product is rounded to fp32 once
    codes = np.array([[0x39]], dtype=np.uint8)  # 1.125
    s = np.array([np.float32(0.1)], dtype=np.float32)
    assert codecs.dequant_fp8(codes, s)[0, 0] == float(np.float32(1.125) * np.float32(0.1))


def test_dequant_mxfp4_nibbles_and_scale():
    # row of 64 elements: bytes hold (even low, odd high)
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21   # element 0 -> code 1 (0.5), element 1 -> code 2 (1.0)
    packed[0, 16] = 0xF7  # element 32 -> code 7 (6.0), element 33 -> code 15 (-6.0)
    e = np.array([[127 + 3, 127 - 1]], dtype=np.uint8)
    out = codecs.dequant_mxfp4(packed, e)
    assert out[0, 0] == 0.5 * 8 and out[0, 1] == 1.0 * 8
    assert out[0, 32] == 6.0 * 0.5 and out[0, 33] == -6.0 * 0.5
    assert np.count_nonzero(out) == 4


def test_bf16_bits():
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-3], dtype=torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


# ---------------------------------------------------------------- mutation tests
# Each plants one plausible mistake in a copy of an oracle routine and checks
# that the pins above notice it.

def _attend_no_scale(q, K, V, scale):
    return attention.attend(q, K, V, 1.0)


def _attend_no_max(q, K, V, scale):
    O, L = attention.attend(q, K, V, scale)
    s = (np.asarray(K, float) @ np.asarray(q, float).T) * scale
    return O, L - s.max(axis=0) if len(K) else L


def _attend_wrong_sign(q, K, V, scale):
    return attention.attend(q, K, V, -scale)


def _attend_transposed_group(q, K, V, scale):
    O, L = attention.attend(q, K, V, scale)
    return O[::-1], L[::-1]


def _combine_linear_weights(Op, Lp):
    w = np.where(np.isneginf(Lp), 0.0, Lp)
    return (w[..., None] * Op).sum(0) / w.sum(0)[..., None], Lp.max(0)


def _combine_unnormalised(Op, Lp):
    m = Lp.max(0)
    w = np.exp(Lp - m)
    return (w[..., None] * Op).sum(0), m + np.log(w.sum(0))


def _combine_drops_max(Op, Lp):
    return attention.combine(Op, Lp)[0], np.log(np.exp(Lp).sum(0) / len(Lp))


def _slot_blockwise(t, P):
    return (t // 16) // P % P, t


def _slot_one_based(t, P):
    return placement.slot(t + 1, P)


@pytest.mark.parametrize("mutant", [_attend_no_scale, _attend_no_max, _attend_wrong_sign, _attend_transposed_group])
def test_mutant_attention_is_caught(mutant):
    with pytest.raises(AssertionError):
        check_bruteforce(mutant)
        check_closed_forms(mutant)


@pytest.mark.parametrize("mutant", [_combine_linear_weights, _combine_unnormalised, _combine_drops_max])
def test_mutant_combine_is_caught(mutant):
    with pytest.raises(AssertionError):
        for seed in range(5):
            check_split_invariance(attention.attend, mutant, seed, 50, 4)


def _partials_slice_slip(q, K, V, scale, P):
    Op, Lp = attention.slice_partials(q, K, V, scale, P)
    return np.roll(Op, 1, axis=0), np.roll(Lp, 1, axis=0)


def _partials_blockwise_mask(q, K, V, scale, P):
    n = K.shape[0]
    O = np.empty((P, q.shape[0], V.shape[1]))
    L = np.empty((P, q.shape[0]))
    for r in range(P):      # contiguous blocks instead of the 16-token rotation
        idx = np.arange(n)[(np.arange(n) * P) // max(n, 1) == r]
        O[r], L[r] = attention.attend(q, K[idx], V[idx], scale)
    return O, L


@pytest.mark.parametrize("mutant", [_partials_slice_slip, _partials_blockwise_mask])
def test_mutant_slice_partials_is_caught(mutant):
    with pytest.raises(AssertionError):
        check_slice_partials(mutant)


@pytest.mark.parametrize("mutant", [_slot_blockwise, _slot_one_based])
def test_mutant_placement_is_caught(mutant, golden_dir):
    with open(os.path.join(golden_dir, "placement_two_slices.json")) as f:
        golden = json.load(f)
    with pytest.raises(AssertionError):
        check_page_placement(mutant, golden)
        check_placement_bijection(mutant)


def test_mutant_codec_is_caught(golden_dir):
    with open(os.path.join(golden_dir, "ocp_formats.json")) as f:
        golden = json.load(f)
    bias8 = np.array([codecs.fp8_e4m3_value(c) / 2 for c in range(256)])
    with pytest.raises(AssertionError):
        check_codec_spec(bias8, codecs.E2M1, codecs.E8M0, golden)
    swapped = codecs.E2M1.copy()
    swapped[[3, 5]] = swapped[[5, 3]]
    with pytest.raises(AssertionError):
        check_codec_spec(codecs.FP8_E4M3, swapped, codecs.E8M0, golden)
