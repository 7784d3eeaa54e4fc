"""Parity of the quantising append (hx_kv_append_bf16) with the oracle's
encoders and open-chunk policy (oracle/quantize.py): bit-exact codes and
scales, read back through hx_kv_dequant, after a prefill and a run of decode
steps and multi-token appends; then a decode step over the quantised cache
against the oracle's attention on the oracle's own codes."""

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
from oracle import placement as opl
from oracle import quantize as oq
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()
    assert torch.cuda.is_available(), "these tests need the GPU"
    yield
    torch.cuda.synchronize()


def _values(B, Hkv, n, D, seed):
    """bf16 rows whose magnitude changes from token to token (so fp8 groups
    raise their scale), with some all-zero rows."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(B, Hkv, n, D, generator=g) * torch.exp2(torch.randint(-3, 1, (B, Hkv, n, 1), generator=g).float())
    zero = torch.rand(B, Hkv, n, 1, generator=g) < 0.05
    x = torch.where(zero, torch.zeros_like(x), x)
    return x.to(torch.bfloat16)


def _calls(ctx, seed):
    """(pos, count) per call: a prefill of part of each request, then decode
    steps of one token and appends of up to 40 tokens (some requests idle)."""
    rng = np.random.default_rng(seed)
    done = [int(rng.integers(0, n // 2 + 1)) for n in ctx]
    calls = [([0] * len(ctx), list(done))]
    while any(d < n for d, n in zip(done, ctx)):
        step = 1 if rng.random() < 0.6 else int(rng.integers(2, 41))
        cnt = [min(step, n - d) if rng.random() < 0.85 else 0 for d, n in zip(done, ctx)]
        if sum(cnt) == 0:
            continue
        calls.append((list(done), cnt))
        done = [d + c for d, c in zip(done, cnt)]
    return calls


def _oracle_fp8(x, ctx, calls):
    """Codes [B, Hkv, n, D] and per-token scales [B, Hkv, n] after the calls."""
    B, Hkv, n, D = x.shape
    xf = x.float().numpy()
    codes = np.zeros((B, Hkv, n, D), dtype=np.uint8)
    scales = np.ones((B, Hkv, (n + 15) // 16), dtype=np.float32)
    for pos, cnt in calls:
        for b in range(B):
            p0, p1 = pos[b], pos[b] + cnt[b]
            t = p0
            while t < p1:
                c = t // 16
                row0 = 16 * c
                hi = min(p1, row0 + 16)
                for g in range(Hkv):
                    chunk = np.zeros((16, D), dtype=np.uint8)
                    m = min(n - row0, 16)
                    chunk[:m] = codes[b, g, row0:row0 + m]
                    new, s = oq.append_fp8_chunk(chunk, scales[b, g, c], t - row0, xf[b, g, t:hi])
                    codes[b, g, row0:row0 + m] = new[:m]
                    scales[b, g, c] = s
                t = hi
    tok_scale = np.repeat(scales, 16, axis=-1)[..., :n]
    return codes, tok_scale


def _oracle_mxfp4(x):
    B, Hkv, n, D = x.shape
    packed, E = oq.quantize_mxfp4_rows(x.float().numpy().reshape(-1, D))
    return packed.reshape(B, Hkv, n, D // 2), E.reshape(B, Hkv, n, D // 32)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


CASES = [
    configs.FP8_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 400), P=4),
    configs.MXFP4_RAGGED.scaled(B=3, Hkv=2, Hq=8, ctx_range=(1, 400), P=4),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.dtype)
def test_quantising_append_matches_oracle(w):
    ctx = synth.context_lengths(w, 21)
    nmax = max(ctx)
    x = _values(w.B, w.Hkv, nmax, w.Dk, seed=22)
    xv = _values(w.B, w.Hkv, nmax, w.Dv, seed=23)
    calls = _calls(ctx, seed=24)
    H.log(f"[quant-append] {w.dtype} ctx={ctx} calls={len(calls)}")
    cap = synth.capacity(ctx, w.P)
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=False, dtype=w.dtype, cap=cap)
    cache = api.KVCache(desc, device=DEV, fill=0xFF)
    kd, vd = x.to(DEV), xv.to(DEV)
    for pos, cnt in calls:
        step = max(cnt)
        kn = torch.stack([torch.nn.functional.pad(kd[b, :, pos[b]:pos[b] + cnt[b]], (0, 0, 0, step - cnt[b]))
                          for b in range(w.B)]).contiguous()
        vn = torch.stack([torch.nn.functional.pad(vd[b, :, pos[b]:pos[b] + cnt[b]], (0, 0, 0, step - cnt[b]))
                          for b in range(w.B)]).contiguous()
        api.kv_append_bf16(cache, kn, vn, pos=pos, count=cnt)
    torch.cuda.synchronize()

    if w.dtype == "fp8_e4m3":
        kc, ks = _oracle_fp8(x, ctx, calls)
        vc, vs = _oracle_fp8(xv, ctx, calls)
        inp = synth.Inputs(w=w, seed=0, ctx=ctx, cap=cap, q=None, k=torch.from_numpy(kc), v=torch.from_numpy(vc),
                           k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs))
    else:
        kc, ke = _oracle_mxfp4(x)
        vc, ve = _oracle_mxfp4(xv)
        inp = synth.Inputs(w=w, seed=0, ctx=ctx, cap=cap, q=None, k=torch.from_numpy(kc), v=torch.from_numpy(vc),
                           k_scale=torch.from_numpy(ke), v_scale=torch.from_numpy(ve))
    # stored bytes, read back through the library's bit-exact decoder
    for b in range(w.B):
        for g in range(w.Hkv):
            K, V = H.token_values(inp, b, g)
            for r in range(w.P):
                toks = opl.slice_tokens(ctx[b], w.P, r)
                if not toks:
                    continue
                ko = torch.empty(len(toks), w.Dk, dtype=torch.float32, device=DEV)
                vo = torch.empty(len(toks), w.Dv, dtype=torch.float32, device=DEV)
                api.kv_dequant(cache, r, b, g, 0, len(toks), ko, vo)
                kr = K[toks].astype(np.float32)
                vr = V[toks].astype(np.float32)
                assert np.array_equal(_bits(ko.cpu().numpy()), _bits(kr)), f"K rows of b={b} g={g} slice={r}"
                assert np.array_equal(_bits(vo.cpu().numpy()), _bits(vr)), f"V rows of b={b} g={g} slice={r}"

    # a decode step over the quantised cache against the oracle on its own codes
    gq = torch.Generator(device=DEV).manual_seed(25)
    inp.q = (torch.randn(w.B, w.Hq, w.Dk, generator=gq, device=DEV)).to(torch.bfloat16)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"quantised {w.dtype}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


def test_bf16_cache_append_is_plain_placement():
    w = configs.TINY_GQA.scaled(B=2, Hkv=2, Hq=4, ctx=None, ctx_range=(1, 200), P=3)
    ctx = synth.context_lengths(w, 5)
    x = _values(w.B, w.Hkv, max(ctx), w.Dk, seed=6).to(DEV)
    xv = _values(w.B, w.Hkv, max(ctx), w.Dv, seed=7).to(DEV)
    cap = synth.capacity(ctx, w.P)
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=False, dtype="bf16", cap=cap)
    a = api.KVCache(desc, device=DEV, fill=0xFF)
    b = api.KVCache(desc, device=DEV, fill=0xFF)
    api.kv_append_bf16(a, x, xv, pos=[0] * w.B, count=ctx)
    api.kv_append(b, x, xv, None, None, pos=[0] * w.B, count=ctx)
    torch.cuda.synchronize()
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


STEP_CASES = [
    # (workload, n_new, steps, layout): narrow and wide groups, dense and block pool
    (configs.FP8_GQA.scaled(B=3, Hkv=2, Hq=8, ctx=None, ctx_range=(1, 300), P=4), 1, 40, "dense"),
    (configs.FP8_GQA.scaled(B=2, Hkv=1, Hq=16, ctx=None, ctx_range=(1, 300), P=8), 1, 20, "paged"),
    (configs.FP8_GQA.scaled(B=2, Hkv=2, Hq=64, ctx=None, ctx_range=(1, 300), P=4), 3, 12, "paged"),
    (configs.MXFP4_RAGGED.scaled(B=3, Hkv=2, Hq=8, ctx_range=(1, 300), P=4), 1, 40, "dense"),
    (configs.MXFP4_RAGGED.scaled(B=2, Hkv=1, Hq=16, ctx_range=(1, 300), P=8), 5, 8, "paged"),
    (configs.MXFP4_RAGGED.scaled(B=2, Hkv=1, Hq=64, ctx_range=(1, 300), P=4), 17, 4, "dense"),
]


def _step_ids(x):
    return x.dtype + f"-G{x.G}" if hasattr(x, "dtype") else str(x)


@pytest.mark.parametrize("w,n_new,steps,layout", STEP_CASES, ids=_step_ids)
def test_quantising_decode_steps_match_oracle(w, n_new, steps, layout):
    """hx_decode_step_bf16 over a run of decode steps (every request gains
    n_new bf16 rows per step, quantised inside the partial kernel): at every
    step its O and LSE are bit-identical to hx_kv_append_bf16 followed by
    hx_decode_attn on a second cache, and the two caches are byte-identical;
    at the end the stored codes and scales are bit-exact with the oracle's
    encoders and open-group policy, and the last step matches the oracle's
    attention."""
    prefill = synth.context_lengths(w, 31)
    final = [p + steps * n_new for p in prefill]
    nmax = max(final)
    x = _values(w.B, w.Hkv, nmax, w.Dk, seed=32)
    xv = _values(w.B, w.Hkv, nmax, w.Dv, seed=33)
    kd, vd = x.to(DEV), xv.to(DEV)
    cap = synth.capacity(final, w.P)
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=False, dtype=w.dtype, cap=cap)
    H.log(f"[quant step] {_step_ids(w)} {layout} n_new={n_new} steps={steps} prefill={prefill}")

    def make():
        if layout == "paged":
            c = api.KVPool(desc, sum(-(-api.slice_len(n, w.P, r) // 16) for n in final for r in range(w.P)),
                           device=DEV, fill=0xFF)
            for b, n in enumerate(final):
                c.reserve(b, n)
            c.table_host[c.table_host >= 0] = np.random.default_rng(34).permutation(c.table_host[c.table_host >= 0])
            c.sync()
            return c
        return api.KVCache(desc, device=DEV, fill=0xFF)

    fused, ref = make(), make()
    app = api.kv_append_bf16_paged if layout == "paged" else api.kv_append_bf16
    attn = api.decode_attn_paged if layout == "paged" else api.decode_attn
    step = api.decode_step_bf16_paged if layout == "paged" else api.decode_step_bf16
    for c in (fused, ref):
        app(c, kd, vd, pos=[0] * w.B, count=prefill)
    gq = torch.Generator(device=DEV).manual_seed(35)
    q = torch.randn(w.B, w.Hq, w.Dk, generator=gq, device=DEV).to(torch.bfloat16)
    ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device=DEV)
    o1 = torch.empty(w.B, w.Hq, w.Dv, device=DEV)
    l1 = torch.empty(w.B, w.Hq, device=DEV)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    planes = lambda c: [t for t in (c.k, c.v, c.k_scale, c.v_scale) if t is not None]
    done = list(prefill)
    calls = [([0] * w.B, list(prefill))]
    for s in range(steps):
        ctx = [d + n_new for d in done]
        kn = torch.stack([kd[b, :, done[b]:ctx[b]] for b in range(w.B)]).contiguous()
        vn = torch.stack([vd[b, :, done[b]:ctx[b]] for b in range(w.B)]).contiguous()
        step(fused, kn, vn, q, ctx, w.softmax_scale, o2, l2, ws)
        app(ref, kn, vn, pos=done, count=[n_new] * w.B)
        attn(ref, q, ctx, w.softmax_scale, o1, l1, ws)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), f"O differs at step {s}"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"LSE differs at step {s}"
        for a_, b_ in zip(planes(ref), planes(fused)):
            assert torch.equal(a_, b_), f"caches differ at step {s}"
        calls.append((list(done), [n_new] * w.B))
        done = ctx

    # the stored bytes against the oracle's encoders (read back bit-exactly)
    if w.dtype == "fp8_e4m3":
        kc, ks = _oracle_fp8(x, done, calls)
        vc, vs = _oracle_fp8(xv, done, calls)
    else:
        (kc, ks), (vc, vs) = _oracle_mxfp4(x), _oracle_mxfp4(xv)
    inp = synth.Inputs(w=w, seed=0, ctx=done, cap=cap, q=q, k=torch.from_numpy(kc), v=torch.from_numpy(vc),
                       k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs))
    deq = api.kv_dequant_paged if layout == "paged" else api.kv_dequant
    for b in range(w.B):
        for g in range(w.Hkv):
            K, V = H.token_values(inp, b, g)
            for r in range(w.P):
                toks = opl.slice_tokens(done[b], w.P, r)
                if not toks:
                    continue
                ko = torch.empty(len(toks), w.Dk, dtype=torch.float32, device=DEV)
                vo = torch.empty(len(toks), w.Dv, dtype=torch.float32, device=DEV)
                deq(fused, r, b, g, 0, len(toks), ko, vo)
                assert np.array_equal(_bits(ko.cpu().numpy()), _bits(K[toks].astype(np.float32))), (b, g, r)
                assert np.array_equal(_bits(vo.cpu().numpy()), _bits(V[toks].astype(np.float32))), (b, g, r)
    oc, lc = o2.cpu().numpy(), l2.cpu().numpy()
    heads = np.arange(w.G)
    for b in range(w.B):
        for g in range(w.Hkv):
            _, _, O, L = H.oracle_group(inp, b, g, heads)
            H.compare(f"quant step b={b} g={g}", oc[b, g * w.G:(g + 1) * w.G], lc[b, g * w.G:(g + 1) * w.G], O, L,
                      w.dtype)
