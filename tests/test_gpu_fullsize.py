"""Parity at the workloads' full sizes (1M-token contexts; ragged up to 2M),
in the launch configuration bench.py times: the cache holds n-1 tokens, the
step appends token n-1, runs the partial kernel over every slice and the
combine.  The oracle checks sampled (request, KV head) groups over their whole
context, per slice and combined."""

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


CASES = [
    (configs.LLAMA405B_SHARE, False, "ends"),
    (configs.LLAMA405B_SHARE, True, "ends"),
    (configs.FP8_GQA, False, "ends"),
    (configs.FP8_GQA, True, "ends"),
    (configs.MXFP4_RAGGED, False, "short_long"),
    (configs.MXFP4_RAGGED, True, "short_long"),
    (configs.DEEPSEEK_MLA, False, "ends"),
    (configs.DEEPSEEK_MLA, True, "ends"),
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
