"""GQA groups of more than 16 query heads per KV head (the wide-group kernel:
tile pairs through an LDS ring, every wave owning its own 16-head blocks),
for every cache format, dense and block pool, against the oracle.

Bars as in test_gpu_parity: O within 2e-3 (bf16 KV) or 2e-2 (fp8 / MXFP4
KV, oracle on the dequantised values) absolute and 1e-2 / 5e-2 relative to
max |O|; LSE within 1e-4 relative; pool partials bit-identical to the dense
cache's."""

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()
    assert torch.cuda.is_available(), "these tests need the GPU"
    yield
    torch.cuda.synchronize()


def _ids(w):
    c = w.ctx if w.ctx is not None else f"{w.ctx_range[0]}-{w.ctx_range[1]}"
    return f"{w.dtype}-B{w.B}-G{w.G}-Hkv{w.Hkv}-P{w.P}-n{c}"


_BASE = {"bf16": configs.LLAMA405B_SHARE, "fp8_e4m3": configs.FP8_GQA, "mxfp4": configs.MXFP4_RAGGED}
# (G, Hkv, B, P, context range): odd widths, several KV heads, tiny contexts
# with empty slices, many splits per slice, the widest group
_SHAPES = [
    (17, 1, 3, 4, (1, 5000)),
    (24, 2, 2, 8, (100, 30000)),
    (32, 1, 3, 8, (1, 40)),
    (64, 1, 2, 8, (20000, 60000)),
    (128, 1, 2, 4, (1, 9000)),
]
WIDE_CASES = [_BASE[dt].scaled(Hq=G * Hkv, Hkv=Hkv, B=B, P=P, ctx=None, ctx_range=rng)
              for dt in ("bf16", "fp8_e4m3", "mxfp4") for (G, Hkv, B, P, rng) in _SHAPES]


def _heads(w):
    """Query heads of a group that the oracle checks: all up to 32, else
    both ends of every 16-head block."""
    if w.G <= 32:
        return np.arange(w.G)
    return np.array(sorted({x for blk in range(0, w.G, 16) for x in (blk, min(blk + 15, w.G - 1))}))


@pytest.mark.parametrize("w", WIDE_CASES, ids=_ids)
def test_wide_group_matches_oracle(w):
    """Slice partials, their combine and the one-call step against the oracle
    (with needles, so every slice's and chunk's rows carry weight)."""
    seed = 50 + len(_ids(w)) + w.G
    H.log(f"[wide] {_ids(w)} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    cache = H.build_cache(inp)
    o_part, lse_part, ws = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    o1 = torch.full_like(o, float("nan"))
    l1 = torch.full_like(lse, float("nan"))
    api.decode_attn(cache, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
    torch.cuda.synchronize()
    heads = _heads(w)
    worst = H.check_step(inp, o_part, lse_part, o, lse, heads=heads, label=_ids(w))
    H.check_step(inp, o_part, lse_part, o1, l1, heads=heads, label=_ids(w) + " one-call")
    H.log(f"   ctx={inp.ctx} worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


def _pool_of(inp, fill=0xFF, seed=0):
    """A block pool holding every request's tokens, each request's blocks
    shuffled among themselves."""
    w = inp.w
    desc = H.desc_of(inp)
    need = sum(-(-api.slice_len(n, w.P, r) // 16) for n in inp.ctx for r in range(w.P))
    pool = api.KVPool(desc, need + 7, device=DEV, fill=fill)
    rng = np.random.default_rng(seed)
    for b, n in enumerate(inp.ctx):
        pool.reserve(b, n)
        sel = pool.table_host[b] >= 0
        pool.table_host[b][sel] = rng.permutation(pool.table_host[b][sel])
    pool.sync()
    api.kv_append_paged(pool, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=inp.ctx)
    return pool


@pytest.mark.parametrize("w", WIDE_CASES, ids=_ids)
def test_wide_group_block_pool_equals_dense(w):
    """The block-pool cache (blocks shuffled) gives partials bit-identical to
    the dense cache's, and its one-call step matches the oracle."""
    seed = 70 + len(_ids(w)) + w.G
    H.log(f"[wide pool] {_ids(w)} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    dense = H.build_cache(inp)
    pool = _pool_of(inp, seed=seed)
    od, ld, ws = H.run_partials(inp, dense)
    op = torch.full_like(od, float("nan"))
    lp = torch.full_like(ld, float("nan"))
    api.decode_attn_partial_paged(pool, inp.q, inp.ctx, w.softmax_scale, op, lp, ws)
    o1 = torch.full((w.B, w.Hq, w.Dv), float("nan"), device=DEV)
    l1 = torch.full((w.B, w.Hq), float("nan"), device=DEV)
    api.decode_attn_paged(pool, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
    torch.cuda.synchronize()
    assert torch.equal(od.view(torch.int32), op.view(torch.int32)), "pool partials differ from the dense cache's"
    assert torch.equal(ld.view(torch.int32), lp.view(torch.int32))
    heads = _heads(w)
    oc, lc = o1.cpu().numpy(), l1.cpu().numpy()
    for b, g in [(b, g) for b in sorted({0, w.B - 1}) for g in range(w.Hkv)]:
        _, _, O, L = H.oracle_group(inp, b, g, heads)
        cols = g * w.G + heads
        H.compare(f"wide pool {_ids(w)} b={b} g={g}", oc[b, cols], lc[b, cols], O, L, w.dtype)


def _slice_row_to_token(j, r, P):
    return ((j // 16) * P + r) * 16 + j % 16


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3", "mxfp4"])
def test_wide_group_score_jumps(dtype):
    """Rows whose scores jump far above everything before them, late in a
    split, for heads in different 16-head blocks of a 128-head group (so
    different waves and, with two blocks per wave, both blocks of a wave):
    the softmax reference must move and the accumulators rescale."""
    w = _BASE[dtype].scaled(Hq=128, Hkv=1, B=1, ctx=120000, ctx_range=None, P=2)

    def plant(b, kb, q):
        def put(j, r, h, target):
            t = _slice_row_to_token(j, r, w.P)
            qh = q[b, h].float()
            alpha = target / (w.softmax_scale * float(qh.norm()))
            kb[0, t] = alpha * qh / qh.norm()

        for i, (j, r) in enumerate(((40, 0), (1000, 1), (1530, 0), (22100, 1), (3000, 0), (50000, 1))):
            put(j, r, (0, 17, 63, 64, 100, 127)[i], (4.0, 8.0, 30.0, 60.0, 5.0, 45.0)[i])
        for j, target in ((100, 3.0), (300, 6.0), (700, 20.0), (5000, 60.0)):   # a staircase for one head
            put(j + 7, 0, 90, target)

    H.log(f"[wide jumps] {dtype}")
    inp = synth.make_inputs(w, 29, device=DEV, plant=plant)
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, heads=np.array([0, 17, 63, 64, 90, 100, 127, 5, 45]),
                         label=f"wide jumps {dtype}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


STEP_CASES = [
    (configs.LLAMA405B_SHARE.scaled(Hq=64, B=2, ctx=None, ctx_range=(20000, 60000)), 1, "dense"),
    (configs.LLAMA405B_SHARE.scaled(Hq=48, Hkv=2, B=3, ctx=None, ctx_range=(40, 9000)), 17, "paged"),
    (configs.FP8_GQA.scaled(Hq=128, B=2, ctx=None, ctx_range=(40, 9000)), 5, "dense"),
    (configs.FP8_GQA.scaled(Hq=24, B=3, ctx=None, ctx_range=(40, 9000)), 1, "paged"),
    (configs.MXFP4_RAGGED.scaled(Hq=32, B=2, ctx_range=(40, 9000)), 3, "dense"),
]


@pytest.mark.parametrize("w,n_new,layout", STEP_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_wide_group_fused_step(w, n_new, layout):
    """hx_decode_step with wide groups: the cache it leaves is byte-identical
    to hx_kv_append's, O and LSE bit-identical to append + hx_decode_attn."""
    seed = 90 + w.G + n_new
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    desc = H.desc_of(inp)
    before = [n - n_new for n in inp.ctx]
    newest = lambda t: None if t is None else torch.stack([t[b, :, n - n_new:n] for b, n in enumerate(inp.ctx)]).contiguous()
    new = [newest(t) for t in (inp.k, inp.v, inp.k_scale, inp.v_scale)]
    caches = []
    for _ in range(2):
        if layout == "paged":
            need = sum(-(-api.slice_len(n, w.P, r) // 16) for n in inp.ctx for r in range(w.P))
            c = api.KVPool(desc, need, device=DEV, fill=0xFF)
            for b, n in enumerate(inp.ctx):
                c.reserve(b, n)
            c.sync()
            api.kv_append_paged(c, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=before)
        else:
            c = api.KVCache(desc, device=DEV, fill=0xFF)
            api.kv_append(c, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=before)
        caches.append(c)
    ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device=DEV)
    o1 = torch.full((w.B, w.Hq, w.Dv), float("nan"), device=DEV)
    l1 = torch.full((w.B, w.Hq), float("nan"), device=DEV)
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    H.log(f"[wide step] G={w.G} {w.dtype} {layout} n_new={n_new} ctx={inp.ctx}")
    if layout == "paged":
        api.kv_append_paged(caches[0], *new, pos=before)
        api.decode_attn_paged(caches[0], inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
        api.decode_step_paged(caches[1], *new, inp.q, inp.ctx, w.softmax_scale, o2, l2, ws)
    else:
        api.kv_append(caches[0], *new, pos=before)
        api.decode_attn(caches[0], inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
        api.decode_step(caches[1], *new, inp.q, inp.ctx, w.softmax_scale, o2, l2, ws)
    torch.cuda.synchronize()
    planes = lambda c: [t for t in (c.k, c.v, c.k_scale, c.v_scale) if t is not None]
    for a, b in zip(planes(caches[0]), planes(caches[1])):
        assert torch.equal(a, b), "the fused append wrote different bytes"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)) and torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    heads = _heads(w)
    oc, lc = o2.cpu().numpy(), l2.cpu().numpy()
    for b, g in [(b, g) for b in sorted({0, w.B - 1}) for g in range(w.Hkv)]:
        _, _, O, L = H.oracle_group(inp, b, g, heads)
        cols = g * w.G + heads
        H.compare(f"wide step b={b} g={g}", oc[b, cols], lc[b, cols], O, L, w.dtype)
