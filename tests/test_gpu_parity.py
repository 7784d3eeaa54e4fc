"""Parity of the HIP path (through the C ABI) with the CPU oracle, at sizes the
oracle finishes in seconds that still span several chunk tiles, several
splits per slice and ragged tails.

Bars: placement and dequantisation bit-exact; O within 2e-3 (bf16 KV) or
2e-2 (fp8 / MXFP4 KV, oracle on the dequantised values) absolute and 1e-2 /
5e-2 relative to max |O|; LSE within 1e-4 relative (helpers.TOL)."""

import dataclasses

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
from oracle import attention as oatt
from oracle import codecs as ocod
from oracle import placement as opl
from tests import helpers as H

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()
    assert torch.cuda.is_available(), "these tests need the GPU"
    yield
    torch.cuda.synchronize()


def _bits_f32(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _same_f32(a, b):
    """Bit-exact equality of fp32 arrays, any NaN matching any NaN."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(_bits_f32(a)[~na], _bits_f32(b)[~nb])


# ---------------------------------------------------------------- cache writes and reads

def _random_storage(w, ctx, seed):
    """Arbitrary storage-format bytes (every bit pattern, NaN codes included)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    nmax = max(ctx)
    kb = {"bf16": 2 * w.Dk, "fp8_e4m3": w.Dk, "mxfp4": w.Dk // 2}[w.dtype]
    vb = {"bf16": 2 * w.Dv, "fp8_e4m3": w.Dv, "mxfp4": w.Dv // 2}[w.dtype]
    rnd = lambda *s: torch.randint(0, 256, s, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    k = rnd(w.B, w.Hkv, nmax, kb)
    v = None if w.v_alias_k else rnd(w.B, w.Hkv, nmax, vb)
    if w.dtype == "bf16":
        k = k.view(torch.bfloat16)
        v = None if v is None else v.view(torch.bfloat16)
    ks = vs = None
    if w.dtype == "fp8_e4m3":
        # one positive scale per 16-token group, repeated per token
        grp = torch.rand(w.B, w.Hkv, -(-nmax // 16), generator=g, device=DEV) * 4 + 0.01
        ks = grp.repeat_interleave(16, dim=-1)[..., :nmax].contiguous()
        vs = (grp * 0.5).repeat_interleave(16, dim=-1)[..., :nmax].contiguous()
    elif w.dtype == "mxfp4":
        ks = torch.randint(100, 160, (w.B, w.Hkv, nmax, w.Dk // 32), generator=g, device=DEV,
                           dtype=torch.int32).to(torch.uint8)
        vs = torch.randint(100, 160, (w.B, w.Hkv, nmax, w.Dv // 32), generator=g, device=DEV,
                           dtype=torch.int32).to(torch.uint8)
    cap = synth.capacity(ctx, w.P)
    return synth.Inputs(w=w, seed=seed, ctx=list(ctx), cap=cap, q=torch.zeros(w.B, w.Hq, w.Dk, dtype=torch.bfloat16,
                                                                                device=DEV),
                        k=k, v=v, k_scale=ks, v_scale=vs)


def _oracle_rows(inp, b, g):
    """Oracle-decoded values of every token of (b, g) as float32 (bf16 by bits)."""
    w = inp.w
    n = inp.ctx[b]
    if w.dtype == "bf16":
        kb = inp.k[b, g, :n].cpu().view(torch.int16).numpy().view(np.uint16)
        K = (kb.astype(np.uint32) << 16).view(np.float32)
        V = None if w.v_alias_k else (inp.v[b, g, :n].cpu().view(torch.int16).numpy().view(np.uint16)
                                      .astype(np.uint32) << 16).view(np.float32)
        if w.v_alias_k:
            V = K[:, :w.Dv]
        return K, V
    K, V = H.token_values(inp, b, g)
    # MXFP4 values beyond the fp32 range (E = 254 with magnitudes 2 to 6) become +-inf, as the fp32 dequantisation gives
    with np.errstate(over="ignore"):
        return K.astype(np.float32), V.astype(np.float32)


def _check_placement(inp, cache):
    w = inp.w
    for b in range(w.B):
        for g in range(w.Hkv):
            K, V = _oracle_rows(inp, b, g)
            for r in range(w.P):
                toks = opl.slice_tokens(inp.ctx[b], w.P, r)
                if not toks:
                    continue
                ko = torch.empty(len(toks), w.Dk, dtype=torch.float32, device=DEV)
                vo = torch.empty(len(toks), w.Dv, dtype=torch.float32, device=DEV)
                api.kv_dequant(cache, r, b, g, 0, len(toks), ko, vo)
                assert _same_f32(ko.cpu().numpy(), K[toks]), f"K rows of slice {r}, b={b}, g={g}"
                assert _same_f32(vo.cpu().numpy(), V[toks]), f"V rows of slice {r}, b={b}, g={g}"


PLACEMENT_CASES = [
    configs.TINY_GQA.scaled(B=2, Hkv=2, Hq=4, ctx=None, ctx_range=(1, 300), P=3),
    configs.FP8_GQA.scaled(B=3, Hkv=1, ctx=None, ctx_range=(1, 400), P=4),
    configs.MXFP4_RAGGED.scaled(B=3, Hkv=2, Hq=4, ctx_range=(1, 500), P=8),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 200), P=2),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 200), P=2, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 200), P=3, dtype="mxfp4"),
]


@pytest.mark.parametrize("w", PLACEMENT_CASES, ids=lambda w: w.dtype + ("-mla" if w.v_alias_k else ""))
def test_append_places_bit_exact(w):
    H.log(f"[placement] {w}")
    ctx = synth.context_lengths(w, 11)
    inp = _random_storage(w, ctx, seed=5)
    cache = H.build_cache(inp)
    _check_placement(inp, cache)


@pytest.mark.parametrize("w", PLACEMENT_CASES[:3], ids=lambda w: w.dtype)
def test_incremental_append_equals_bulk(w):
    H.log(f"[incremental] {w}")
    ctx = synth.context_lengths(w, 3)
    inp = _random_storage(w, ctx, seed=9)
    bulk = H.build_cache(inp)
    desc = H.desc_of(inp)
    inc = api.KVCache(desc, device=DEV, fill=0xFF)
    rng = np.random.default_rng(0)
    done = [0] * w.B
    while any(d < n for d, n in zip(done, ctx)):
        step = int(rng.integers(1, 40))
        counts = [min(step, n - d) if rng.random() < 0.8 else 0 for d, n in zip(done, ctx)]
        if sum(counts) == 0:
            continue
        sl = lambda t, b: t[b:b + 1, :, done[b]:done[b] + step] if t is not None else None
        # one call per step; each request's rows start at its own position
        kn = torch.stack([torch.nn.functional.pad(inp.k[b, :, done[b]:done[b] + counts[b]].view(torch.uint8),
                                                  (0, 0, 0, step - counts[b])) for b in range(w.B)])
        vn = None if inp.v is None else torch.stack(
            [torch.nn.functional.pad(inp.v[b, :, done[b]:done[b] + counts[b]].view(torch.uint8),
                                     (0, 0, 0, step - counts[b])) for b in range(w.B)])
        if w.dtype == "bf16":
            kn, vn = kn.view(torch.bfloat16), vn.view(torch.bfloat16)
        ksn = vsn = None
        if inp.k_scale is not None:
            padfn = (lambda t, c: torch.nn.functional.pad(t, (0, step - c))) if w.dtype == "fp8_e4m3" else \
                (lambda t, c: torch.nn.functional.pad(t, (0, 0, 0, step - c)))
            ksn = torch.stack([padfn(inp.k_scale[b, :, done[b]:done[b] + counts[b]], counts[b]) for b in range(w.B)])
            vsn = torch.stack([padfn(inp.v_scale[b, :, done[b]:done[b] + counts[b]], counts[b]) for b in range(w.B)])
        api.kv_append(inc, kn.contiguous(), None if vn is None else vn.contiguous(),
                      None if ksn is None else ksn.contiguous(), None if vsn is None else vsn.contiguous(),
                      pos=done, count=counts)
        done = [d + c for d, c in zip(done, counts)]
        del sl
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(bulk, name), getattr(inc, name)
        if a is not None:
            assert torch.equal(a, b), f"plane {name} differs"


def test_fp8_every_code_dequantises_exactly():
    w = configs.FP8_GQA.scaled(B=1, ctx=32, P=2)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(16).reshape(32, 128)
    scales = torch.tensor([0.5] * 16 + [3.0] * 16, dtype=torch.float32)
    inp = synth.Inputs(w=w, seed=0, ctx=[32], cap=16, q=torch.zeros(1, 16, 128, dtype=torch.bfloat16, device=DEV),
                       k=codes[None, None].to(DEV), v=codes.flip(0)[None, None].contiguous().to(DEV),
                       k_scale=scales[None, None].to(DEV), v_scale=(scales * 0.25)[None, None].to(DEV))
    cache = H.build_cache(inp)
    _check_placement(inp, cache)
    # NaN codes decode to NaN; 0x7E is 448
    assert np.isnan(ocod.FP8_E4M3[0x7F]) and ocod.FP8_E4M3[0x7E] == 448.0


def test_mxfp4_every_code_and_exponent_dequantises_exactly():
    w = configs.MXFP4_RAGGED.scaled(B=1, ctx=None, ctx_range=(48, 48), P=2)
    pairs = torch.arange(256, dtype=torch.int32).to(torch.uint8)    # every (low, high) nibble pair
    packed = pairs.repeat(48 * 64 // 256).reshape(48, 64)
    exps = torch.tensor([1, 64, 120, 127, 134, 200, 254, 255], dtype=torch.int32).to(torch.uint8)
    e8 = exps.repeat(48 * 4 // 8).reshape(48, 4)
    inp = synth.Inputs(w=w, seed=0, ctx=[48], cap=32, q=torch.zeros(1, 16, 128, dtype=torch.bfloat16, device=DEV),
                       k=packed[None, None].to(DEV), v=packed.flip(1)[None, None].contiguous().to(DEV),
                       k_scale=e8[None, None].to(DEV), v_scale=e8.flip(0)[None, None].contiguous().to(DEV))
    cache = H.build_cache(inp)
    _check_placement(inp, cache)


def test_fp8_open_group_keeps_its_stored_scale():
    """Storage-format append into an fp8 group that already holds rows: the
    group keeps its stored scale (the new tokens' scales are not used), so
    the earlier rows decode as before; a group whose first row is new takes
    the scale of that row."""
    w = configs.FP8_GQA.scaled(B=1, Hkv=1, Hq=4, ctx=None, ctx_range=(40, 40), P=2)
    g = torch.Generator(device=DEV).manual_seed(77)
    codes = torch.randint(0, 0x7F, (1, 1, 40, w.Dk), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    vcodes = torch.randint(0, 0x7F, (1, 1, 40, w.Dv), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    s1 = torch.full((1, 1, 40), 0.5, device=DEV)
    s2 = torch.full((1, 1, 40), 3.0, device=DEV)
    inp = synth.Inputs(w=w, seed=0, ctx=[40], cap=synth.capacity([40], w.P), q=torch.zeros(1, 4, w.Dk, dtype=torch.bfloat16,
                                                                                            device=DEV),
                       k=codes, v=vcodes, k_scale=s1, v_scale=s1)
    cache = H.build_cache(inp, upto=[5])                                  # rows 0-4 of group 0 with scale 0.5
    tail = lambda t: t[:, :, 5:].clone()                  # source row i is token 5 + i (fresh, aligned)
    api.kv_append(cache, tail(codes), tail(vcodes), tail(s2), tail(s2), pos=[5], count=[30])   # tokens 5-34
    torch.cuda.synchronize()
    ko = torch.empty(24, w.Dk, device=DEV)
    vo = torch.empty(24, w.Dv, device=DEV)
    api.kv_dequant(cache, 0, 0, 0, 0, 24, ko, vo)          # slice 0: group 0 (rows 0-15), group 2 (rows 16-23 = tokens 32-39)
    expect_k = ocod.dequant_fp8(codes[0, 0].cpu().numpy(), np.array([0.5, 0.5, 3.0], dtype=np.float32))
    expect_v = ocod.dequant_fp8(vcodes[0, 0].cpu().numpy(), np.array([0.5, 0.5, 3.0], dtype=np.float32))
    rows = opl.slice_tokens(35, w.P, 0)                     # tokens held by slice 0 after 35 tokens
    assert _same_f32(ko[:len(rows)].cpu().numpy(), expect_k[rows].astype(np.float32))
    assert _same_f32(vo[:len(rows)].cpu().numpy(), expect_v[rows].astype(np.float32))
    ko1 = torch.empty(16, w.Dk, device=DEV)
    api.kv_dequant(cache, 1, 0, 0, 0, 16, ko1, None)       # slice 1: group 1 (tokens 16-31), first row new: scale 3
    torch.cuda.synchronize()
    expect_k1 = ocod.dequant_fp8(codes[0, 0, 16:32].cpu().numpy(), np.array([3.0], dtype=np.float32))
    assert _same_f32(ko1.cpu().numpy(), expect_k1.astype(np.float32))


def test_fp8_zero_scales_in_the_last_tile():
    """A zero K or V scale is a valid encoding (all values 0).  In the last,
    partial tile of a slice the masked rows must not turn it into NaN: the
    scores of a zero-K-scale group are 0, and a zero-V-scale group adds
    weight but no value."""
    w = configs.FP8_GQA.scaled(B=3, ctx=None, ctx_range=(1000, 3000), P=4)
    inp = synth.make_inputs(w, 61, device=DEV, needles=True)
    for b, n in enumerate(inp.ctx):
        last = (n - 1) // 16 * 16                          # first token of the last (partial) group
        if b in (0, 2):
            inp.k_scale[b, :, last:n] = 0.0
        if b in (1, 2):
            inp.v_scale[b, :, last:n] = 0.0
        inp.k_scale[b, :, 160:176] = 0.0                   # and one full group inside a slice
    H.log(f"[fp8 zero scales] ctx={inp.ctx}")
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label="fp8 zero scales")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


@pytest.mark.parametrize("hq", [16, 64, 128], ids=["G16", "G64", "G128"])
def test_mxfp4_value_scales_over_a_wide_exponent_range(hq):
    """The V block scales of an MXFP4 cache enter the value product through
    the exponent fields of the bf16 weights (an integer add, no multiply):
    with the block exponents spread over 2^-60 .. 2^30 of the quantiser's,
    every output row must stay within the format's relative bound of the
    oracle's (O then spans many orders of magnitude, so the bound is taken
    against each group's largest |O|), and the LSE is untouched."""
    w = configs.MXFP4_RAGGED.scaled(B=2, Hq=hq, ctx_range=(3000, 9000), P=4)
    inp = synth.make_inputs(w, 77, device=DEV, needles=True)
    gen = torch.Generator().manual_seed(5)
    shift = torch.randint(-60, 31, tuple(inp.v_scale.shape), generator=gen, dtype=torch.int16)
    inp.v_scale = (inp.v_scale.cpu().to(torch.int16) + shift).clamp(1, 254).to(torch.uint8).to(DEV)
    H.log(f"[mxfp4 wide exponents] G={w.G} ctx={inp.ctx}")
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    oc, lc = o.cpu().numpy(), lse.cpu().numpy()
    for b, g in H.all_groups(inp):
        _, _, O, L = H.oracle_group(inp, b, g)
        cols = g * w.G + np.arange(w.G)
        rel = float(np.max(np.abs(oc[b, cols] - O)) / np.max(np.abs(O)))
        lrel = float(np.max(np.abs(lc[b, cols] - L) / np.maximum(1.0, np.abs(L))))
        H.log(f"   b={b} g={g} max|O|={np.max(np.abs(O)):.2e} |dO|/max|O|={rel:.2e} LSE rel={lrel:.2e}")
        assert np.all(np.isfinite(oc[b, cols]))
        assert rel <= H.TOL["mxfp4"]["rel_o"] and lrel <= H.LSE_REL


# ---------------------------------------------------------------- attention parity

PARITY_CASES = [
    configs.TINY_GQA,                                                                     # the tiny config itself
    configs.TINY_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 6000), P=4),        # GQA G=4, ragged
    configs.LLAMA405B_SHARE.scaled(B=2, ctx=None, ctx_range=(1, 40000)),                  # G=16, P=8
    configs.LLAMA405B_SHARE.scaled(B=3, ctx=None, ctx_range=(1, 50), P=2),                # tiny contexts
    configs.FP8_GQA.scaled(B=3, ctx=None, ctx_range=(100, 20000)),
    configs.MXFP4_RAGGED.scaled(B=3, ctx_range=(1, 30000)),
    configs.LLAMA405B_SHARE.scaled(B=2, Hq=2, ctx=None, ctx_range=(100, 9000), P=5),      # G=2
    configs.TINY_GQA.scaled(B=1, Hq=1, ctx=3333, P=1),                                     # P=1, G=1
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4),                 # MLA, ragged
    configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(1, 40), P=8),                   # MLA, empty slices
    configs.DEEPSEEK_MLA.scaled(B=1, ctx=20011, P=2),                                     # MLA, many splits
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4, dtype="fp8_e4m3"),   # quantised MLA
    configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(1, 40), P=8, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=1, ctx=20011, P=2, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4, dtype="mxfp4"),
    configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(1, 40), P=8, dtype="mxfp4"),
    configs.DEEPSEEK_MLA.scaled(B=1, ctx=20011, P=2, dtype="mxfp4"),
]


def _ids(w):
    c = w.ctx if w.ctx is not None else f"{w.ctx_range[0]}-{w.ctx_range[1]}"
    return f"{w.dtype}-B{w.B}-G{w.G}-Hkv{w.Hkv}-P{w.P}-n{c}"


@pytest.mark.parametrize("needles", [False, True], ids=["plain", "needles"])
@pytest.mark.parametrize("w", PARITY_CASES, ids=_ids)
def test_decode_step_matches_oracle(w, needles):
    seed = 1 + len(_ids(w))
    H.log(f"[parity] {_ids(w)} needles={needles} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV, needles=needles)
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=_ids(w))
    H.log(f"   ctx={inp.ctx} worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


def _slice_row_to_token(j, r, P):
    """Token index of local row j of slice r (the inverse of the placement)."""
    return ((j // 16) * P + r) * 16 + j % 16


@pytest.mark.parametrize("staircase", [False, True], ids=["one-jump", "staircase"])
def test_mla_large_score_jumps(staircase):
    """Scores far above everything seen earlier in a run of tiles (more than
    2^64 in base 2): the MLA kernel keeps the first tile's max as its softmax
    reference and must start the run over with a larger one.  Rows aligned
    with one head's query get natural-log scores of 50-160, placed past the
    first tiles of runs in both slices, for heads served by different waves;
    the staircase raises one head's score three times within one run."""
    w = configs.DEEPSEEK_MLA.scaled(B=1, ctx=200000, P=2)
    inp = synth.make_inputs(w, 17, device=DEV)
    k = inp.k[0, 0]                             # [n, 576] bf16

    def plant(j, r, h, target):
        t = _slice_row_to_token(j, r, w.P)
        qh = inp.q[0, h].float()
        alpha = target / (w.softmax_scale * float(qh.norm()))
        k[t] = (alpha * qh / qh.norm()).to(torch.bfloat16)

    if staircase:
        for r, h in ((0, 0), (1, 77)):
            for j, target in ((100, 50.0), (300, 100.0), (700, 160.0)):
                plant(j, r, h, target)
    else:
        for i, (j, r) in enumerate(((40, 0), (100, 1), (1530, 0), (2210, 1), (3000, 0), (60000, 1))):
            plant(j, r, (0, 45, 77, 127, 33, 100)[i], 60.0)
    H.log(f"[jumps] staircase={staircase}")
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"jumps staircase={staircase}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


@pytest.mark.parametrize("staircase", [False, True], ids=["one-jump", "staircase"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3", "mxfp4"])
def test_gqa_score_jumps(dtype, staircase):
    """Rows whose scores rise far above everything before them, late in a
    split: the GQA kernel moves a head's softmax reference only when a tile
    raises it (bf16) or raises it by more than 2^8 (fp8, MXFP4), so jumps
    both below and above that margin are planted.  Rows aligned with one
    head's query get natural-log scores of 3-60; the staircase raises the
    same heads four times within one split."""
    w = configs.LLAMA405B_SHARE.scaled(B=1, ctx=200000, P=2, dtype=dtype)

    def plant(b, kb, q):
        def put(j, r, h, target):
            t = _slice_row_to_token(j, r, w.P)
            qh = q[b, h].float()
            alpha = target / (w.softmax_scale * float(qh.norm()))
            kb[0, t] = alpha * qh / qh.norm()

        if staircase:
            for r, h in ((0, 0), (1, 9), (0, 15)):
                for j, target in ((100, 3.0), (300, 6.0), (700, 20.0), (5000, 60.0)):
                    put(j + h, r, h, target)
        else:
            for i, (j, r) in enumerate(((40, 0), (1000, 1), (1530, 0), (22100, 1), (3000, 0), (60000, 1))):
                put(j, r, (0, 4, 7, 11, 13, 15)[i], (4.0, 8.0, 30.0, 60.0, 5.0, 45.0)[i])

    H.log(f"[gqa jumps] {dtype} staircase={staircase}")
    inp = synth.make_inputs(w, 23, device=DEV, plant=plant)
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"gqa jumps {dtype} staircase={staircase}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


def test_mla_value_product_precision():
    """Short slices, where a few weights dominate: with P split into a bf16
    high part and residual (default) the MLA output is within ~1e-5 of the
    oracle over all 128 heads; with HX_FLAG_P_BF16 (P rounded once) the
    error is of the order 2^-8 times V's spread, still within 2e-3 here."""
    w = configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(1, 40), P=8)
    inp = synth.make_inputs(w, 40, device=DEV)
    worst = {}
    for flags in (0, api.HX_FLAG_P_BF16):
        desc = dataclasses.replace(H.desc_of(inp), flags=flags)
        cache = api.KVCache(desc, device=DEV, fill=0xFF)
        api.kv_append(cache, inp.k, None, None, None, pos=[0] * w.B, count=inp.ctx)
        o_part, lse_part, _ = H.run_partials(inp, cache)
        o, lse = H.run_combine(o_part, lse_part)
        torch.cuda.synchronize()
        worst[flags] = H.check_step(inp, o_part, lse_part, o, lse, label=f"mla flags={flags}")[0]
    H.log(f"   worst |dO| split P {worst[0]:.2e}, P rounded once {worst[1]:.2e}")
    assert worst[0] <= 2e-5 < worst[1]


@pytest.mark.parametrize("needles", [False, True], ids=["plain", "needles"])
def test_mla_long_runs_skip_residual_products(monkeypatch, needles):
    """One workgroup per slice streams 1,024 tiles, so past its first tiles
    every weight is below 2^-10 of its head's running sum and the kernel
    skips the residual products of P; tiles holding needles keep them.  The
    output stays within the bf16 bound of the oracle over all 128 heads, and
    close to the oracle in absolute terms (many small rounding errors)."""
    monkeypatch.setenv("HX_MIN_CHUNKS_PER_WG", "4096")     # one split per slice
    w = configs.DEEPSEEK_MLA.scaled(B=1, ctx=65536, P=2)
    inp = synth.make_inputs(w, 41, device=DEV, needles=needles)
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"mla long runs needles={needles}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")
    assert worst[0] <= 2e-4


def test_partials_are_deterministic_and_workspace_reusable():
    w = configs.LLAMA405B_SHARE.scaled(B=2, ctx=None, ctx_range=(5000, 60000))
    inp = synth.make_inputs(w, 4, device=DEV)
    cache = H.build_cache(inp)
    o1, l1, ws = H.run_partials(inp, cache)
    # a different, smaller problem through the same workspace in between
    w2 = configs.TINY_GQA.scaled(B=2, Hq=16, P=8, ctx=None, ctx_range=(1, 3000))
    inp2 = synth.make_inputs(w2, 5, device=DEV)
    cache2 = H.build_cache(inp2)
    big = torch.zeros(max(ws.numel(), api.workspace_size(cache2.desc, w2.Hq)), dtype=torch.uint8, device=DEV)
    a_o, a_l, _ = H.run_partials(inp, cache, big)
    b_o, b_l, _ = H.run_partials(inp2, cache2, big)
    c_o, c_l, _ = H.run_partials(inp, cache, big)
    torch.cuda.synchronize()
    assert torch.equal(o1, a_o) and torch.equal(a_o, c_o)
    assert torch.equal(l1, a_l) and torch.equal(a_l, c_l)
    H.check_step(inp2, b_o, b_l, *H.run_combine(b_o, b_l), label="reused workspace")
    H.check_step(inp, c_o, c_l, *H.run_combine(c_o, c_l), groups=[(0, 0)], label="after reuse")


def test_decode_step_append_then_attend():
    """The bench's step: the cache holds n-1 tokens, the step appends token
    n-1 and attends over n; repeating the step is idempotent."""
    w = configs.LLAMA405B_SHARE.scaled(B=3, ctx=None, ctx_range=(2, 20000))
    inp = synth.make_inputs(w, 8, device=DEV, needles=True)
    cache = H.build_cache(inp, upto=[n - 1 for n in inp.ctx])
    last = [n - 1 for n in inp.ctx]
    kn = torch.stack([inp.k[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()
    vn = torch.stack([inp.v[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()
    for _ in range(2):
        api.kv_append(cache, kn, vn, None, None, pos=last)
        o_part, lse_part, _ = H.run_partials(inp, cache)
        o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    H.check_step(inp, o_part, lse_part, o, lse, label="append+attend")


ONE_CALL_CASES = [
    configs.TINY_GQA,
    configs.TINY_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 6000), P=4),
    configs.FP8_GQA.scaled(B=2, ctx=None, ctx_range=(100, 9000)),
    configs.MXFP4_RAGGED.scaled(B=2, ctx_range=(1, 9000)),
    configs.LLAMA405B_SHARE.scaled(B=2, ctx=None, ctx_range=(20000, 60000)),      # many splits per slice
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4, dtype="mxfp4"),
]


@pytest.mark.parametrize("w", ONE_CALL_CASES, ids=_ids)
def test_decode_attn_whole_step(w):
    """hx_decode_attn (partials, then one fold of every slice's partial or
    split records into the final output) against the oracle's unsplit
    attention; three calls on one workspace give identical bits."""
    seed = 3 + len(_ids(w))
    H.log(f"[one-call] {_ids(w)} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    cache = H.build_cache(inp)
    ws = torch.zeros(api.workspace_size(cache.desc, w.Hq), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        o = torch.full((w.B, w.Hq, w.Dv), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=DEV)
        api.decode_attn(cache, inp.q, inp.ctx, w.softmax_scale, o, lse, ws)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    o, lse = outs[0]
    oc, lc = o.cpu().numpy(), lse.cpu().numpy()
    worst = [0.0, 0.0]
    for b, g in H.all_groups(inp):
        heads = np.arange(w.G) if w.G <= 16 else np.array([0, 31, 32, 63, 64, 95, 96, 127])
        _, _, O, L = H.oracle_group(inp, b, g, heads)
        cols = g * w.G + heads
        e = H.compare(f"{_ids(w)} b={b} g={g}", oc[b, cols], lc[b, cols], O, L, w.dtype)
        worst = [max(worst[0], e[0]), max(worst[1], e[1])]
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


EDGE_CASES = [
    configs.TINY_GQA.scaled(B=70, Hkv=1, Hq=3, ctx=None, ctx_range=(1, 200), P=3),        # B > 64: two launches, G=3
    configs.TINY_GQA.scaled(B=2, Hkv=8, Hq=8, ctx=None, ctx_range=(1, 3000), P=64),       # P = 64, G = 1, 8 KV heads
    configs.FP8_GQA.scaled(B=66, Hkv=2, Hq=10, ctx=None, ctx_range=(1, 300), P=2),       # fp8, G = 5, two launches
    configs.MXFP4_RAGGED.scaled(B=65, Hkv=1, Hq=7, ctx_range=(1, 500), P=5),              # MXFP4, G = 7, two launches
    configs.LLAMA405B_SHARE.scaled(B=2, Hkv=2, Hq=32, ctx=None, ctx_range=(3000, 30000)),   # G = 16 with 2 KV heads
    configs.DEEPSEEK_MLA.scaled(B=66, ctx=None, ctx_range=(1, 100), P=1),                 # MLA, P = 1, two launches
    configs.DEEPSEEK_MLA.scaled(B=66, ctx=None, ctx_range=(1, 100), P=1, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=5, ctx=None, ctx_range=(1, 33), P=64, dtype="mxfp4"),   # quantised MLA, P = 64
]


@pytest.mark.parametrize("w", EDGE_CASES, ids=_ids)
def test_edge_shapes(w):
    """Batches that take several launches, the largest slice count, odd and
    unit group widths, several KV heads of 16 query heads each, MLA with one
    slice: partials, combine and the one-call step against the oracle."""
    seed = 5 + len(_ids(w))
    H.log(f"[edge] {_ids(w)} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    cache = H.build_cache(inp)
    o_part, lse_part, ws = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    o1 = torch.full_like(o, float("nan"))
    l1 = torch.full_like(lse, float("nan"))
    api.decode_attn(cache, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
    torch.cuda.synchronize()
    heads = [0, 31, 64, 127] if w.Hq == 128 else None
    groups = H.all_groups(inp) if w.B * w.Hkv <= 16 else [(b, g) for b in (0, 1, 63, 64, w.B - 1) for g in range(w.Hkv)]
    worst = H.check_step(inp, o_part, lse_part, o, lse, groups=groups, heads=heads, label=_ids(w))
    H.check_step(inp, o_part, lse_part, o1, l1, groups=groups, heads=heads, label=_ids(w) + " one-call")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


@pytest.mark.parametrize("P", [1, 3, 8, 100])
def test_lse_combine_matches_oracle(P):
    g = torch.Generator(device="cpu").manual_seed(P)
    B, Hq, Dv = 3, 5, 128
    o_part = torch.randn(P, B, Hq, Dv, generator=g)
    lse_part = torch.randn(P, B, Hq, generator=g) * 20
    empty = torch.rand(P, B, Hq, generator=g) < 0.3
    lse_part[empty] = float("-inf")
    o_part[empty] = 0.0
    lse_part[:, 0, 0] = float("-inf")      # an all-empty row
    o_part[:, 0, 0] = 0.0
    o, lse = H.run_combine(o_part.to(DEV), lse_part.to(DEV))
    O, L = oatt.combine(o_part.double().numpy(), lse_part.double().numpy())
    torch.cuda.synchronize()
    oc, lc = o.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lc), np.isneginf(L))
    fin = ~np.isneginf(L)
    assert np.max(np.abs(lc[fin] - L[fin]) / np.maximum(1, np.abs(L[fin]))) <= 1e-6
    assert np.max(np.abs(oc - O)) <= 1e-5
    assert np.all(oc[0, 0] == 0)
