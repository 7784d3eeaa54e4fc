"""Seeded synthetic inputs for a decode workload.

This module only draws random tensors and writes them in the cache's storage
formats; it holds none of the attention arithmetic and shares nothing with
the HIP library or the oracle, both of which consume what it produces.

Recipe (seed s):
  1. ragged context lengths: torch CPU generator seeded with s, integers
     uniform in [lo, hi] inclusive, drawn first;
  2. a generator on the target device seeded with s draws, in order, Q
     (fp32 N(0, std^2) -> bf16, round to nearest even), then for every
     request its K and then its V (fp32 N(0, std^2));
  3. optional needles: for each query head h, a few rows of its KV head at
     fixed places (first row, 16-row and slice-round boundaries, middle, last
     rows) are replaced by k = a * q_h / |q_h| with a chosen so those rows
     hold about half of head h's softmax mass;
  4. storage format: bf16 (round to nearest even); fp8 e4m3 with one fp32
     scale per 16-token group, scale = amax / 448 (1 when amax = 0), codes =
     round-to-nearest-even of clamp(x / scale, +-448); MXFP4 with one e8m0
     exponent E = clamp(floor(log2 amax) - 2, -127, 127) + 127 per 32
     elements of a row and e2m1 codes = x / 2^(E-127) rounded to nearest
     (ties to even) on the e2m1 grid, saturating at +-6, two codes per byte
     with the even element in the low nibble.
"""

import math
from dataclasses import dataclass
from typing import List, Optional

import torch

from .configs import Workload

CHUNK = 16
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


@dataclass
class Inputs:
    w: Workload
    seed: int
    ctx: List[int]
    cap: int                       # rows per slice plane
    q: torch.Tensor                # bf16 [B, Hq, Dk]
    k: torch.Tensor                # storage format, token-major [B, Hkv, nmax, ...]
    v: Optional[torch.Tensor]
    k_scale: Optional[torch.Tensor]   # fp8: f32 [B, Hkv, nmax] (the group's scale per token); mxfp4: u8 [B, Hkv, nmax, D/32]
    v_scale: Optional[torch.Tensor]
    needles: Optional[dict] = None    # head -> list of token positions

    @property
    def nmax(self):
        return max(self.ctx)


def context_lengths(w: Workload, seed: int) -> List[int]:
    if w.ctx is not None:
        return [w.ctx] * w.B
    lo, hi = w.ctx_range
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64).tolist()


def capacity(ctx: List[int], P: int) -> int:
    per = -(-max(ctx) // (CHUNK * P))
    return max(1, per) * CHUNK


def needle_positions(n: int, P: int, G: int) -> dict:
    """Rows replaced by needles, per head of a KV group (distinct rows)."""
    base = [0, CHUNK - 1, CHUNK, CHUNK * P - 1, CHUNK * P, n // 2, n - CHUNK - 1, n - 1]
    taken, out = set(), {}
    for hh in range(G):
        mine = []
        for t in base:
            t = min(max(t + hh, 0), n - 1)
            if t not in taken:
                taken.add(t)
                mine.append(t)
        out[hh] = mine
    return out


def _quant_fp8(x):
    """x fp32 [..., n, D] -> (codes u8 [..., n, D], per-token group scale f32 [..., n])."""
    n, D = x.shape[-2], x.shape[-1]
    ng = -(-n // CHUNK)
    pad = ng * CHUNK - n
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    xg = xp.reshape(*x.shape[:-2], ng, CHUNK * D)
    amax = xg.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    codes = (xg / scale[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = codes.reshape(*x.shape[:-2], ng * CHUNK, D)[..., :n, :]
    tok_scale = scale.repeat_interleave(CHUNK, dim=-1)[..., :n]
    return codes.contiguous(), tok_scale.contiguous()


def _quant_mxfp4(x):
    """x fp32 [..., n, D] -> (packed u8 [..., n, D/2], e8m0 u8 [..., n, D/32])."""
    D = x.shape[-1]
    xb = x.reshape(*x.shape[:-1], D // 32, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.floor(torch.log2(amax)) - 2.0                # -inf for amax = 0
    e = e.clamp(-127.0, 127.0)
    E = (e + 127.0).to(torch.int32)
    y = xb / torch.exp2(e)[..., None]
    a = y.abs()
    idx = torch.zeros_like(a, dtype=torch.int32)
    mids = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
    for i, t in enumerate(mids):                            # ties go to the even code
        idx += ((a > t) | ((a == t) & (i % 2 == 1))).to(torch.int32)
    code = idx | ((y < 0) & (idx > 0)).to(torch.int32) << 3
    code = code.reshape(*x.shape[:-1], D).to(torch.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), E.to(torch.uint8).contiguous()


def _store(x, dtype):
    if dtype == "bf16":
        return x.to(torch.bfloat16), None
    if dtype == "fp8_e4m3":
        return _quant_fp8(x)
    return _quant_mxfp4(x)


def make_inputs(w: Workload, seed: int = 0, device="cuda", needles: bool = False, plant=None) -> Inputs:
    """Seeded inputs of workload w.  `plant(b, kb, q)`, if given, may edit the
    fp32 K rows kb [Hkv, n, Dk] of request b (before they are stored in the
    cache format), e.g. to set rows with chosen scores."""
    ctx = context_lengths(w, seed)
    nmax = max(ctx)
    cap = capacity(ctx, w.P)
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    q32 = torch.randn(w.B, w.Hq, w.Dk, generator=g, device=dev) * w.std
    q = q32.to(torch.bfloat16)
    kd = {"bf16": (w.Dk,), "fp8_e4m3": (w.Dk,), "mxfp4": (w.Dk // 2,)}[w.dtype]
    vd = {"bf16": (w.Dv,), "fp8_e4m3": (w.Dv,), "mxfp4": (w.Dv // 2,)}[w.dtype]
    cdt = torch.bfloat16 if w.dtype == "bf16" else torch.uint8
    k = torch.zeros(w.B, w.Hkv, nmax, *kd, dtype=cdt, device=dev)
    v = None if w.v_alias_k else torch.zeros(w.B, w.Hkv, nmax, *vd, dtype=cdt, device=dev)
    ks = vs = None
    if w.dtype == "fp8_e4m3":
        ks = torch.ones(w.B, w.Hkv, nmax, dtype=torch.float32, device=dev)
        vs = None if w.v_alias_k else torch.ones_like(ks)
    elif w.dtype == "mxfp4":
        ks = torch.full((w.B, w.Hkv, nmax, w.Dk // 32), 127, dtype=torch.uint8, device=dev)
        vs = None if w.v_alias_k else torch.full((w.B, w.Hkv, nmax, w.Dv // 32), 127, dtype=torch.uint8, device=dev)
    needle_map = {} if needles else None
    G = w.G
    for b in range(w.B):
        n = ctx[b]
        kb = torch.randn(w.Hkv, n, w.Dk, generator=g, device=dev) * w.std
        vb = None if w.v_alias_k else torch.randn(w.Hkv, n, w.Dv, generator=g, device=dev) * w.std
        if needles:
            pos = needle_positions(n, w.P, G)
            # The other rows' scores are about N(0, sigma_s^2), so they sum to about
            # n exp(sigma_s^2 / 2); a needle score of ln(n / count) + sigma_s^2 / 2
            # gives the needles about half of the mass.
            sigma_s = w.std * w.std * math.sqrt(w.Dk) * w.softmax_scale
            for gg in range(w.Hkv):
                for hh in range(G):
                    h = gg * G + hh
                    qh = q[b, h].to(torch.float32)
                    ts = pos[hh]
                    target = math.log(max(n / max(len(ts), 1), 2.0)) + 0.5 * sigma_s * sigma_s
                    alpha = target / (w.softmax_scale * float(qh.norm()))
                    kb[gg, ts] = (alpha * qh / qh.norm())[None, :]
            needle_map[b] = pos
        if plant is not None:
            plant(b, kb, q)
        kc, kscale = _store(kb, w.dtype)
        k[b, :, :n] = kc
        if ks is not None:
            ks[b, :, :n] = kscale
        if vb is not None:
            vc, vscale = _store(vb, w.dtype)
            v[b, :, :n] = vc
            if vs is not None:
                vs[b, :, :n] = vscale
        del kb, vb
    return Inputs(w=w, seed=seed, ctx=ctx, cap=cap, q=q, k=k, v=v, k_scale=ks, v_scale=vs, needles=needle_map)
