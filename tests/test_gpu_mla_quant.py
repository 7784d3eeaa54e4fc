"""Quantised MLA caches: fp8 e4m3 and MXFP4 latent rows (576 columns, V the
first 512 of the same stored row, one plane of packed tiles).  Placement,
dequantisation, attention, the one-call and fused steps and the block pool
are covered next to the other formats (test_gpu_parity.py,
test_gpu_decode_step.py, test_gpu_pool.py); here: the quantising append and
the quantising decode step of aliased rows, bit-exact against the oracle's
encoders, and scores that force the MLA kernel's restart on quantised rows."""

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
from oracle import placement as opl
from tests import helpers as H
from tests.test_gpu_quant_append import _bits, _calls, _oracle_fp8, _oracle_mxfp4, _values

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()
    assert torch.cuda.is_available(), "these tests need the GPU"
    yield
    torch.cuda.synchronize()


def _oracle_inputs(w, x, ctx, calls, cap):
    """The oracle's stored codes and scales of the latent rows x after the calls."""
    if w.dtype == "fp8_e4m3":
        kc, ks = _oracle_fp8(x, ctx, calls)
    else:
        kc, ks = _oracle_mxfp4(x)
    return synth.Inputs(w=w, seed=0, ctx=ctx, cap=cap, q=None, k=torch.from_numpy(kc), v=None,
                        k_scale=torch.from_numpy(ks), v_scale=None)


def _check_rows(inp, cache, label):
    """Every stored row, read back through hx_kv_dequant, equals the oracle's
    decoding of its own codes bit for bit (K: all 576 columns; V: the first
    512 of the same row)."""
    w = inp.w
    for b in range(w.B):
        K, V = H.token_values(inp, b, 0)
        for r in range(w.P):
            toks = opl.slice_tokens(inp.ctx[b], w.P, r)
            if not toks:
                continue
            ko = torch.empty(len(toks), w.Dk, dtype=torch.float32, device=DEV)
            vo = torch.empty(len(toks), w.Dv, dtype=torch.float32, device=DEV)
            api.kv_dequant(cache, r, b, 0, 0, len(toks), ko, vo)
            assert np.array_equal(_bits(ko.cpu().numpy()), _bits(K[toks].astype(np.float32))), f"{label} K b={b} r={r}"
            assert np.array_equal(_bits(vo.cpu().numpy()), _bits(V[toks].astype(np.float32))), f"{label} V b={b} r={r}"


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "mxfp4"])
def test_mla_quantising_append_matches_oracle(dtype):
    """hx_kv_append_bf16 of 576-wide latent rows over a prefill, decode steps
    and multi-token appends: the stored codes and scales are the oracle's
    (fp8: a 16-row group's scale grows with its rows and the stored codes are
    re-encoded); then the attention over the cache against the oracle."""
    w = configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(1, 400), P=4, dtype=dtype)
    ctx = synth.context_lengths(w, 51)
    x = _values(w.B, w.Hkv, max(ctx), w.Dk, seed=52)
    calls = _calls(ctx, seed=53)
    cap = synth.capacity(ctx, w.P)
    H.log(f"[mla quant-append] {dtype} ctx={ctx} calls={len(calls)}")
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=True, dtype=dtype, cap=cap)
    cache = api.KVCache(desc, device=DEV, fill=0xFF)
    kd = x.to(DEV)
    for pos, cnt in calls:
        step = max(cnt)
        kn = torch.stack([torch.nn.functional.pad(kd[b, :, pos[b]:pos[b] + cnt[b]], (0, 0, 0, step - cnt[b]))
                          for b in range(w.B)]).contiguous()
        api.kv_append_bf16(cache, kn, None, pos=pos, count=cnt)
    torch.cuda.synchronize()
    inp = _oracle_inputs(w, x, ctx, calls, cap)
    _check_rows(inp, cache, f"mla {dtype}")
    gq = torch.Generator(device=DEV).manual_seed(54)
    inp.q = (torch.randn(w.B, w.Hq, w.Dk, generator=gq, device=DEV) * 0.5).to(torch.bfloat16)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"mla quantised {dtype}")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("dtype", ["fp8_e4m3", "mxfp4"])
def test_mla_quantising_decode_steps(dtype, layout):
    """hx_decode_step_bf16 on a quantised MLA cache over a run of steps: at
    every step O and LSE are bit-identical to hx_kv_append_bf16 followed by
    hx_decode_attn on a second cache, the caches stay byte-identical, and at
    the end the rows are the oracle's encodings and the last step matches the
    oracle's attention."""
    w = configs.DEEPSEEK_MLA.scaled(B=2, ctx=None, ctx_range=(1, 300), P=4, dtype=dtype)
    n_new, steps = 2, 12
    prefill = synth.context_lengths(w, 61)
    final = [p + steps * n_new for p in prefill]
    x = _values(w.B, w.Hkv, max(final), w.Dk, seed=62)
    kd = x.to(DEV)
    cap = synth.capacity(final, w.P)
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=True, dtype=dtype, cap=cap)
    H.log(f"[mla quant step] {dtype} {layout} prefill={prefill}")
    caches = []
    for _ in range(2):
        if layout == "paged":
            need = sum(-(-api.slice_len(n, w.P, r) // 16) for n in final for r in range(w.P))
            c = api.KVPool(desc, need, device=DEV, fill=0xFF)
            for b, n in enumerate(final):
                c.reserve(b, n)
            c.sync()
            api.kv_append_bf16_paged(c, kd, None, pos=[0] * w.B, count=prefill)
        else:
            c = api.KVCache(desc, device=DEV, fill=0xFF)
            api.kv_append_bf16(c, kd, None, pos=[0] * w.B, count=prefill)
        caches.append(c)
    gq = torch.Generator(device=DEV).manual_seed(63)
    q = (torch.randn(w.B, w.Hq, w.Dk, generator=gq, device=DEV) * 0.5).to(torch.bfloat16)
    ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device=DEV)
    o1 = torch.empty(w.B, w.Hq, w.Dv, device=DEV)
    l1 = torch.empty(w.B, w.Hq, device=DEV)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    ctx = list(prefill)
    for _ in range(steps):
        pos = list(ctx)
        ctx = [c + n_new for c in ctx]
        kn = torch.stack([kd[b, :, pos[b]:pos[b] + n_new] for b in range(w.B)]).contiguous()
        if layout == "paged":
            api.kv_append_bf16_paged(caches[0], kn, None, pos=pos)
            api.decode_attn_paged(caches[0], q, ctx, w.softmax_scale, o1, l1, ws)
            api.decode_step_bf16_paged(caches[1], kn, None, q, ctx, w.softmax_scale, o2, l2, ws)
        else:
            api.kv_append_bf16(caches[0], kn, None, pos=pos)
            api.decode_attn(caches[0], q, ctx, w.softmax_scale, o1, l1, ws)
            api.decode_step_bf16(caches[1], kn, None, q, ctx, w.softmax_scale, o2, l2, ws)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    for a, b in zip((caches[0].k,), (caches[1].k,)):
        assert torch.equal(a, b), "the step wrote different bytes"
    calls = [([0] * w.B, list(prefill))] + [([p + i * n_new for p in prefill], [n_new] * w.B) for i in range(steps)]
    inp = _oracle_inputs(w, x, ctx, calls, cap)
    inp.q = q
    if layout == "dense":
        _check_rows(inp, caches[1], f"mla step {dtype}")
    heads = np.arange(w.G)
    oc, lc = o2.cpu().numpy(), l2.cpu().numpy()
    for b in range(w.B):
        _, _, O, L = H.oracle_group(inp, b, 0, heads)
        H.compare(f"mla step {dtype} {layout} b={b}", oc[b], lc[b], O, L, dtype)


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "mxfp4"])
def test_mla_quantised_score_jumps_restart(dtype):
    """Rows aligned with one head's query, placed past the first tiles of
    runs, with natural-log scores of 60-160 (far beyond the kernel's 2^64
    headroom over the first tile's max): the run restarts on converted
    quantised rows as on bf16 ones."""
    w = configs.DEEPSEEK_MLA.scaled(B=1, ctx=120000, P=2, dtype=dtype)

    def plant(b, kb, q):
        for j, r, h, target in ((300, 0, 0, 60.0), (900, 1, 77, 100.0), (2500, 0, 127, 160.0)):
            t = ((j // 16) * w.P + r) * 16 + j % 16
            qh = q[b, h].float()
            alpha = target / (w.softmax_scale * float(qh.norm()))
            kb[0, t] = alpha * qh / qh.norm()

    inp = synth.make_inputs(w, 71, device=DEV, plant=plant)
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label=f"mla {dtype} jumps")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")


def test_mla_fp8_zero_group_scales():
    """A zero group scale is a valid fp8 encoding (all values 0): such a
    group's scores are 0 and its rows add weight but no value, so the kernel
    normalises by their unrounded weights.  Zero scales in a full group
    inside a slice and in the partial last group of every request, against
    the oracle on the dequantised values."""
    w = configs.DEEPSEEK_MLA.scaled(B=3, ctx=None, ctx_range=(300, 3000), P=4, dtype="fp8_e4m3")
    inp = synth.make_inputs(w, 73, device=DEV, needles=True)
    for b, n in enumerate(inp.ctx):
        last = (n - 1) // 16 * 16                 # first token of the last group
        inp.k_scale[b, :, last:n] = 0.0
        inp.k_scale[b, :, 160:176] = 0.0          # and one full group inside a slice
    H.log(f"[mla fp8 zero scales] ctx={inp.ctx}")
    cache = H.build_cache(inp)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    worst = H.check_step(inp, o_part, lse_part, o, lse, label="mla fp8 zero scales")
    H.log(f"   worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")
