"""Block-pool (paged) caches on the GPU: rows placed through block tables
that grow over many appends (blocks of different requests and slices
interleaved in the pool, recycled blocks holding stale rows, never-written
bytes set to NaN patterns), read back bit-exactly against the oracle's
token values, and decode partials that are bit-identical to the dense
cache's and match the oracle."""

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
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


def _window(t, b, p0, cnt, n_new):
    """Rows [p0, p0 + cnt) of request b of a token-major tensor, padded to n_new rows."""
    if t is None:
        return None
    x = t[b, :, p0:p0 + cnt]                      # [Hkv, cnt, ...]
    pad = [0, 0] * (x.dim() - 2) + [0, n_new - cnt]   # F.pad lists the last dimension first
    return torch.nn.functional.pad(x, pad)


def _schedule(ctx, seed):
    """(pos, count) per append call: a prefill of part of each request, then
    steps of 1-300 tokens with some requests idle."""
    rng = np.random.default_rng(seed)
    done = [int(rng.integers(0, n // 3 + 1)) for n in ctx]
    calls = [([0] * len(ctx), list(done))]
    while any(d < n for d, n in zip(done, ctx)):
        step = 1 if rng.random() < 0.3 else int(rng.integers(2, 301))
        cnt = [min(step, n - d) if rng.random() < 0.8 else 0 for d, n in zip(done, ctx)]
        if sum(cnt) == 0:
            continue
        calls.append((list(done), cnt))
        done = [d + c for d, c in zip(done, cnt)]
    return calls


def _stale(pool, inp, seed):
    """Fill part of the pool with another request's rows, then give the blocks
    back: later owners find stale, finite rows in them."""
    n = min(max(inp.ctx), 16 * inp.w.P * 6)
    pool.reserve(0, n)
    pool.sync()
    g = torch.Generator(device=DEV).manual_seed(seed)
    w = inp.w
    if w.dtype == "bf16":
        k = (torch.randn(w.B, w.Hkv, n, w.Dk, generator=g, device=DEV)).to(torch.bfloat16)
        v = None if w.v_alias_k else (torch.randn(w.B, w.Hkv, n, w.Dv, generator=g, device=DEV)).to(torch.bfloat16)
        api.kv_append_paged(pool, k, v, None, None, pos=[0] * w.B, count=[n] + [0] * (w.B - 1))
    else:
        k = (torch.randn(w.B, w.Hkv, n, w.Dk, generator=g, device=DEV)).to(torch.bfloat16)
        v = None if w.v_alias_k else (torch.randn(w.B, w.Hkv, n, w.Dv, generator=g, device=DEV)).to(torch.bfloat16)
        api.kv_append_bf16_paged(pool, k, v, pos=[0] * w.B, count=[n] + [0] * (w.B - 1))
    torch.cuda.synchronize()
    pool.release(0)


def build_pool(inp, seed, spare=9):
    """A pool holding inp's rows, written by a growing sequence of appends."""
    w = inp.w
    desc = H.desc_of(inp)
    need = sum(opl.blocks_needed(n, w.P, r) for n in inp.ctx for r in range(w.P))
    pool = api.KVPool(desc, need + spare, device=DEV, fill=0xFF)
    _stale(pool, inp, seed + 100)
    calls = _schedule(inp.ctx, seed)
    for pos, cnt in calls:
        for b in range(w.B):
            pool.reserve(b, pos[b] + cnt[b])
        pool.sync()
        step = max(cnt)
        sel = lambda t: None if t is None else torch.stack([_window(t, b, pos[b], cnt[b], step) for b in range(w.B)])
        api.kv_append_paged(pool, sel(inp.k).contiguous(), None if inp.v is None else sel(inp.v).contiguous(),
                            None if inp.k_scale is None else sel(inp.k_scale).contiguous(),
                            None if inp.v_scale is None else sel(inp.v_scale).contiguous(), pos=pos, count=cnt)
    torch.cuda.synchronize()
    assert pool.free_blocks() == spare
    return pool, len(calls)


CASES = [
    configs.TINY_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 3000), P=4),
    configs.FP8_GQA.scaled(B=2, ctx=None, ctx_range=(1, 5000), P=8),
    configs.MXFP4_RAGGED.scaled(B=3, Hkv=2, Hq=16, ctx_range=(1, 4000), P=3),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4),
    configs.LLAMA405B_SHARE.scaled(B=1, ctx=40000, P=2),                     # many splits per slice
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=4, dtype="fp8_e4m3"),
    configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 3000), P=3, dtype="mxfp4"),
]


def _ids(w):
    c = w.ctx if w.ctx is not None else f"{w.ctx_range[0]}-{w.ctx_range[1]}"
    return f"{w.dtype}-Dk{w.Dk}-B{w.B}-G{w.G}-Hkv{w.Hkv}-P{w.P}-n{c}"


def _bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("w", CASES, ids=_ids)
def test_paged_rows_and_partials(w):
    seed = 3 + len(_ids(w))
    inp = synth.make_inputs(w, seed, device=DEV, needles=True)
    pool, ncalls = build_pool(inp, seed)
    H.log(f"[pool] {_ids(w)} ctx={inp.ctx} appends={ncalls} blocks={pool.num_blocks}")
    # rows, read back through the block table, are the oracle's token values bit for bit
    for b in range(w.B):
        for g in range(w.Hkv):
            K, V = H.token_values(inp, b, g)
            for r in range(w.P):
                toks = opl.slice_tokens(inp.ctx[b], w.P, r)
                L = len(toks)
                if L == 0:
                    continue
                ko = torch.empty(L, w.Dk, dtype=torch.float32, device=DEV)
                vo = None if w.v_alias_k else torch.empty(L, w.Dv, dtype=torch.float32, device=DEV)
                api.kv_dequant_paged(pool, r, b, g, 0, L, ko, vo)
                assert np.array_equal(ko.cpu().numpy().view(np.uint32), K[toks].astype(np.float32).view(np.uint32)), \
                    f"K rows b={b} g={g} r={r}"
                if vo is not None:
                    assert np.array_equal(vo.cpu().numpy().view(np.uint32),
                                          V[toks].astype(np.float32).view(np.uint32)), f"V rows b={b} g={g} r={r}"
    # partials: bit-identical to the dense cache's, and the oracle's
    dense = H.build_cache(inp)
    od, ld, ws = H.run_partials(inp, dense)
    op = torch.empty_like(od)
    lp = torch.empty_like(ld)
    api.decode_attn_partial_paged(pool, inp.q, inp.ctx, w.softmax_scale, op, lp, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(op), _bits(od)) and np.array_equal(_bits(lp), _bits(ld))
    o, lse = H.run_combine(op, lp)
    torch.cuda.synchronize()
    heads = [0, 31, 32, 63, 64, 95, 96, 127] if w.Hq == 128 else None
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    worst = H.check_step(inp, op, lp, o, lse, groups=groups, heads=heads, label=f"pool {_ids(w)}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")
    # the whole step in one call, also bit-identical to the dense cache's
    o1 = torch.empty_like(o)
    l1 = torch.empty_like(lse)
    o2 = torch.empty_like(o)
    l2 = torch.empty_like(lse)
    api.decode_attn(dense, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
    api.decode_attn_paged(pool, inp.q, inp.ctx, w.softmax_scale, o2, l2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o1), _bits(o2)) and np.array_equal(_bits(l1), _bits(l2))


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "mxfp4"])
def test_paged_quantising_append_matches_dense(dtype):
    """The quantising append through a block table writes the bytes the dense
    cache gets, over the same sequence of appends."""
    w = configs.FP8_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 700), P=4, dtype=dtype)
    ctx = synth.context_lengths(w, 31)
    g = torch.Generator(device=DEV).manual_seed(32)
    nmax = max(ctx)
    x = (torch.randn(w.B, w.Hkv, nmax, w.Dk, generator=g, device=DEV) *
         torch.exp2(torch.randint(-3, 1, (w.B, w.Hkv, nmax, 1), generator=g, device=DEV).float())).to(torch.bfloat16)
    xv = (torch.randn(w.B, w.Hkv, nmax, w.Dv, generator=g, device=DEV)).to(torch.bfloat16)
    cap = synth.capacity(ctx, w.P)
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=False, dtype=dtype, cap=cap)
    dense = api.KVCache(desc, device=DEV, fill=0xFF)
    need = sum(opl.blocks_needed(n, w.P, r) for n in ctx for r in range(w.P))
    pool = api.KVPool(desc, need, device=DEV, fill=0xFF)
    calls = _schedule(ctx, 33)
    for pos, cnt in calls:
        for b in range(w.B):
            pool.reserve(b, pos[b] + cnt[b])
        pool.sync()
        step = max(cnt)
        kn = torch.stack([_window(x, b, pos[b], cnt[b], step) for b in range(w.B)]).contiguous()
        vn = torch.stack([_window(xv, b, pos[b], cnt[b], step) for b in range(w.B)]).contiguous()
        api.kv_append_bf16(dense, kn, vn, pos=pos, count=cnt)
        api.kv_append_bf16_paged(pool, kn, vn, pos=pos, count=cnt)
    torch.cuda.synchronize()
    H.log(f"[pool quant-append] {dtype} ctx={ctx} calls={len(calls)}")
    for b in range(w.B):
        for hg in range(w.Hkv):
            for r in range(w.P):
                L = opl.slice_len(ctx[b], w.P, r)
                if L == 0:
                    continue
                outs = []
                for src, fn in ((dense, api.kv_dequant), (pool, api.kv_dequant_paged)):
                    ko = torch.empty(L, w.Dk, dtype=torch.float32, device=DEV)
                    vo = torch.empty(L, w.Dv, dtype=torch.float32, device=DEV)
                    fn(src, r, b, hg, 0, L, ko, vo)
                    outs.append((_bits(ko), _bits(vo)))
                assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_out_of_range_block_ids_stay_inside_the_pool():
    """A table entry outside [0, num_blocks) is clamped on the device: the
    call reads some block of the pool (wrong rows) and completes; with the
    table repaired the next call is right again."""
    w = configs.TINY_GQA.scaled(B=1, Hkv=1, Hq=8, ctx=600, P=2)
    inp = synth.make_inputs(w, 5, device=DEV)
    pool, _ = build_pool(inp, 5, spare=0)
    good = pool.table_host.copy()
    pool.table_host[0, 0, 1] = pool.num_blocks + 1000
    pool.table_host[0, 1, 2] = -7
    pool.sync()
    o_part = torch.empty(w.P, w.B, w.Hq, w.Dv, dtype=torch.float32, device=DEV)
    lse_part = torch.empty(w.P, w.B, w.Hq, dtype=torch.float32, device=DEV)
    ws = torch.zeros(api.workspace_size(pool.desc, w.Hq), dtype=torch.uint8, device=DEV)
    api.decode_attn_partial_paged(pool, inp.q, inp.ctx, w.softmax_scale, o_part, lse_part, ws)
    torch.cuda.synchronize()
    pool.table_host[...] = good
    pool.sync()
    api.decode_attn_partial_paged(pool, inp.q, inp.ctx, w.softmax_scale, o_part, lse_part, ws)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    H.check_step(inp, o_part, lse_part, o, lse, label="pool repaired")
