"""Named decode workloads (shapes only; every input is synthetic).

The shapes follow the models the pages evaluate on (Helix review, Prompt
1.4.1 "Benchmarks & Environment": Llama-405B, dense GQA with 128 query / 8 KV
heads; DeepSeek-R1, MLA with one latent KV head; 1M-token contexts) plus
fp8 / MXFP4 cache variants.  No weights or datasets are involved.
"""

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    v_alias_k: bool
    dtype: str                 # "bf16" | "fp8_e4m3" | "mxfp4"
    P: int                     # KV slices
    ctx: Optional[int]         # uniform context length, or
    ctx_range: Optional[Tuple[int, int]] = None   # ragged: integer uniform in [lo, hi]
    std: float = 1.0           # standard deviation of Q, K, V before quantisation
    scale: Optional[float] = None   # softmax scale; default 1/sqrt(Dk)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def softmax_scale(self):
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.Dk)

    def scaled(self, **kw):
        return replace(self, **kw)


TINY_GQA = Workload("tiny_gqa", B=1, Hq=8, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", P=4, ctx=4096)
LLAMA405B_SHARE = Workload("llama405b_tpa8_share", B=8, Hq=16, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16",
                           P=8, ctx=1 << 20)
DEEPSEEK_MLA = Workload("deepseek_r1_mla", B=8, Hq=128, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="bf16", P=8,
                        ctx=1 << 20, std=0.5)
FP8_GQA = Workload("fp8_gqa", B=32, Hq=16, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="fp8_e4m3", P=8,
                   ctx=1 << 20)
MXFP4_RAGGED = Workload("mxfp4_ragged", B=16, Hq=16, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="mxfp4", P=8,
                        ctx=None, ctx_range=(4096, 2 * 1024 * 1024))

# A wide GQA group (64 query heads on one KV head, e.g. Llama-405B's 128:8
# at TPA = 2): both products dense enough for the matrix cores to matter.
WIDE_GQA_G64 = Workload("wide_gqa_g64", B=8, Hq=64, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", P=8,
                        ctx=1 << 20)

# The MLA step with quantised latent rows (the review's DeepSeek-R1 results
# are for FP4): fp8 e4m3 and MXFP4 caches of the same shape.
DEEPSEEK_MLA_FP8 = DEEPSEEK_MLA.scaled(name="deepseek_r1_mla_fp8", dtype="fp8_e4m3")
DEEPSEEK_MLA_MXFP4 = DEEPSEEK_MLA.scaled(name="deepseek_r1_mla_mxfp4", dtype="mxfp4")

ALL = {w.name: w for w in (TINY_GQA, LLAMA405B_SHARE, DEEPSEEK_MLA, FP8_GQA, MXFP4_RAGGED, WIDE_GQA_G64,
                           DEEPSEEK_MLA_FP8, DEEPSEEK_MLA_MXFP4)}
