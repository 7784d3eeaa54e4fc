"""Parity at the workloads' full sizes (1M-token contexts; ragged up to 2M),
in the launch configurations bench.py times.  The cache holds n-1 tokens and
the step adds token n-1: either as separate calls (append, the partial kernel
over every slice, the combine; checked per slice and combined) or as one
hx_decode_step (bench.py's default step).  The oracle checks sampled
(request, KV head) groups over their whole context."""

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import api, configs, synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()
    yield
    torch.cuda.empty_cache()


def _step(inp):
    w = inp.w
    cache = H.build_cache(inp, fill=0xFF, upto=[n - 1 for n in inp.ctx])
    last = [n - 1 for n in inp.ctx]
    pick = lambda t: None if t is None else torch.stack([t[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()
    api.kv_append(cache, pick(inp.k), pick(inp.v), pick(inp.k_scale), pick(inp.v_scale), pos=last)
    o_part, lse_part, _ = H.run_partials(inp, cache)
    o, lse = H.run_combine(o_part, lse_part)
    torch.cuda.synchronize()
    del cache
    return o_part, lse_part, o, lse


RAGGED_BF16 = configs.MXFP4_RAGGED.scaled(name="ragged_bf16", dtype="bf16")
RAGGED_FP8 = configs.MXFP4_RAGGED.scaled(name="ragged_fp8", dtype="fp8_e4m3")

CASES = [
    (configs.LLAMA405B_SHARE, False, "ends"),
    (configs.LLAMA405B_SHARE, True, "ends"),
    (configs.FP8_GQA, False, "ends"),
    (configs.FP8_GQA, True, "ends"),
    (configs.MXFP4_RAGGED, False, "short_long"),
    (configs.MXFP4_RAGGED, True, "short_long"),
    # the ragged batch in bf16 and fp8: its one-round split plan needs more
    # workgroups than one round holds (each slice's last split is short), so
    # the launch is planned again with more, shorter workgroups, dispatched
    # longest first
    (RAGGED_BF16, False, "short_long"),
    (RAGGED_FP8, True, "short_long"),
    (configs.DEEPSEEK_MLA, False, "ends"),
    (configs.DEEPSEEK_MLA, True, "ends"),
    (configs.DEEPSEEK_MLA_FP8, True, "ends"),
    (configs.DEEPSEEK_MLA_MXFP4, True, "ends"),
    # 64 query heads per KV head: the wide-group kernel, all heads checked
    (configs.WIDE_GQA_G64, True, "ends"),
]

# MLA groups hold 128 query heads: the oracle checks heads at both ends of
# each 32-head block the kernel assigns to one wave pair.
MLA_HEADS = [0, 31, 32, 63, 64, 95, 96, 127]


@pytest.mark.parametrize("w,needles,sample", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_full_size_sampled_groups(w, needles, sample):
    H.log(f"[fullsize] {w.name} needles={needles}: generating")
    inp = synth.make_inputs(w, seed=0, device="cuda", needles=needles)
    H.log(f"[fullsize] {w.name}: ctx min {min(inp.ctx)} max {max(inp.ctx)}; running the step")
    o_part, lse_part, o, lse = _step(inp)
    if sample == "ends":
        groups = [(0, 0), (w.B - 1, w.Hkv - 1)]
    else:
        groups = [(min(range(w.B), key=lambda b: inp.ctx[b]), 0), (max(range(w.B), key=lambda b: inp.ctx[b]), 0)]
    for grp in groups:
        H.log(f"[fullsize] {w.name}: oracle on group {grp} (n={inp.ctx[grp[0]]})")
        heads = MLA_HEADS if w.G == 128 else None
        worst = H.check_step(inp, o_part, lse_part, o, lse, groups=[grp], heads=heads, label=f"{w.name} {grp}")
        H.log(f"[fullsize]    worst |dO|={worst[0]:.2e} LSE rel={worst[1]:.2e}")
    del inp, o_part, lse_part, o, lse
    torch.cuda.empty_cache()


STEP_CASES = [configs.LLAMA405B_SHARE, configs.FP8_GQA, configs.MXFP4_RAGGED, RAGGED_BF16, configs.DEEPSEEK_MLA,
              configs.DEEPSEEK_MLA_MXFP4, configs.WIDE_GQA_G64]


@pytest.mark.parametrize("w", STEP_CASES, ids=lambda x: x.name)
def test_full_size_fused_step(w):
    """bench.py's default step at full size: the cache holds n-1 tokens and
    one hx_decode_step appends token n-1 inside the partial kernel and folds
    the slices.  hx_decode_attn over the cache it leaves must give the same
    bits (the appended rows are what the attention read), and sampled groups
    must match the oracle."""
    H.log(f"[fullsize step] {w.name}: generating")
    inp = synth.make_inputs(w, seed=1, device="cuda", needles=True)
    cache = H.build_cache(inp, fill=0xFF, upto=[n - 1 for n in inp.ctx])
    last = [n - 1 for n in inp.ctx]
    pick = lambda t: None if t is None else torch.stack([t[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()
    ws = torch.zeros(api.workspace_size(H.desc_of(inp), w.Hq), dtype=torch.uint8, device="cuda")
    o1 = torch.full((w.B, w.Hq, w.Dv), float("nan"), device="cuda")
    l1 = torch.full((w.B, w.Hq), float("nan"), device="cuda")
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    H.log(f"[fullsize step] {w.name}: ctx min {min(inp.ctx)} max {max(inp.ctx)}; fused step, then decode_attn")
    api.decode_step(cache, pick(inp.k), pick(inp.v), pick(inp.k_scale), pick(inp.v_scale), inp.q, inp.ctx,
                    w.softmax_scale, o2, l2, ws)
    api.decode_attn(cache, inp.q, inp.ctx, w.softmax_scale, o1, l1, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)) and torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    oc, lc = o2.cpu().numpy(), l2.cpu().numpy()
    del cache, ws
    if w.ctx is None:   # ragged: the shortest and the longest request
        groups = [(min(range(w.B), key=lambda b: inp.ctx[b]), 0), (max(range(w.B), key=lambda b: inp.ctx[b]), 0)]
    else:
        groups = [(0, 0), (w.B - 1, w.Hkv - 1)]
    heads = np.array(MLA_HEADS) if w.G == 128 else np.arange(w.G)
    for b, g in groups:
        H.log(f"[fullsize step] {w.name}: oracle on group {(b, g)} (n={inp.ctx[b]})")
        _, _, O, L = H.oracle_group(inp, b, g, heads)
        cols = g * w.G + heads
        e = H.compare(f"{w.name} fused step b={b} g={g}", oc[b, cols], lc[b, cols], O, L, w.dtype)
        H.log(f"[fullsize step]    |dO|={e[0]:.2e} LSE rel={e[1]:.2e}")
    del inp
    torch.cuda.empty_cache()
