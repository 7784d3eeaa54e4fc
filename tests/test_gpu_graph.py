"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph on the
caller's stream): append + partial attention + combine, and the one-call
form, on dense and block-pool caches.  Every replay, with the program's own
eager work and synchronisations in between, must give the eager step's
output bit for bit.  The library issues no memset and allocates nothing
during a step, so the captured kernels are the whole step."""

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


def _bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


CASES = [
    (configs.TINY_GQA, "dense"),                                                   # one split per slice
    (configs.LLAMA405B_SHARE.scaled(B=2, ctx=None, ctx_range=(20000, 70000)), "dense"),   # split fold inside
    (configs.MXFP4_RAGGED.scaled(B=3, ctx_range=(100, 9000), P=4), "paged"),
    (configs.DEEPSEEK_MLA.scaled(B=1, ctx=9000, P=2), "dense"),
]


@pytest.mark.parametrize("w,layout", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_captured_step_replays_match_eager(w, layout):
    inp = synth.make_inputs(w, 12, device=DEV)
    desc = H.desc_of(inp)
    if layout == "paged":
        need = sum(-(-api.slice_len(n, w.P, r) // 16) for n in inp.ctx for r in range(w.P))
        cache = api.KVPool(desc, need, device=DEV)
        for b, n in enumerate(inp.ctx):
            cache.reserve(b, n)
        cache.sync()
        append, partial, one = api.kv_append_paged, api.decode_attn_partial_paged, api.decode_attn_paged
    else:
        cache = api.KVCache(desc, device=DEV)
        append, partial, one = api.kv_append, api.decode_attn_partial, api.decode_attn
    append(cache, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=[n - 1 for n in inp.ctx])
    last = [n - 1 for n in inp.ctx]
    newest = lambda t: None if t is None else torch.stack([t[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()
    kn, vn, ksn, vsn = newest(inp.k), newest(inp.v), newest(inp.k_scale), newest(inp.v_scale)
    ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device=DEV)
    o_part = torch.empty(w.P, w.B, w.Hq, w.Dv, dtype=torch.float32, device=DEV)
    lse_part = torch.empty(w.P, w.B, w.Hq, dtype=torch.float32, device=DEV)
    o = torch.empty(w.B, w.Hq, w.Dv, dtype=torch.float32, device=DEV)
    lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device=DEV)
    o1 = torch.empty_like(o)
    l1 = torch.empty_like(lse)

    def step(stream):
        append(cache, kn, vn, ksn, vsn, pos=last, stream=stream)
        partial(cache, inp.q, inp.ctx, w.softmax_scale, o_part, lse_part, ws, stream=stream)
        api.lse_combine(o_part, lse_part, o, lse, stream=stream)
        one(cache, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws, stream=stream)

    # eager reference
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [_bits(t) for t in (o_part, lse_part, o, lse, o1, l1)]
    H.log(f"[graph] {w.name} {layout} ctx={inp.ctx}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm the side stream once before capture
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        for t in (o_part, lse_part, o, lse, o1, l1):
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in (o_part, lse_part, o, lse, o1, l1)]
        for name, a, b in zip(("o_part", "lse_part", "o", "lse", "o (one call)", "lse (one call)"), got, ref):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager step"
    H.check_step(inp, o_part, lse_part, o, lse, groups=[(0, 0)],
                 heads=[0, 31, 64, 127] if w.Hq == 128 else None, label=f"graph {w.name}")
