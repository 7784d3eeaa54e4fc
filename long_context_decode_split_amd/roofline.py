"""Algorithmic work of one decode step: KV bytes the method must read once,
and matrix-core flops, with MI355X peaks.

The bandwidth model is the one behind the Helix summary's TP roofline
(paragraph on tensor parallelism: batch 8, 1M tokens, FP4, 1,024 us per layer
at TP=1 falling to 128 us at TP=8 and flat beyond): time = KV bytes read per
GPU / HBM bandwidth, where a GPU holds ceil(K / TP) KV heads but never fewer
than one.
"""

import math

HBM_PEAK_BYTES_PER_S = 8.0e12        # MI355X HBM3E
MFMA_BF16_DENSE_FLOPS = 2.5e15       # MI355X dense bf16 matrix peak
CHUNK = 16


def kv_bytes_per_token(Dk, Dv, v_alias_k, dtype):
    """Bytes of one token row of one KV head: codes plus scales."""
    width = Dk + (0 if v_alias_k else Dv)
    if dtype == "bf16":
        return 2.0 * width
    if dtype == "fp8_e4m3":
        return 1.0 * width + 4.0 / CHUNK * (1 if v_alias_k else 2)
    if dtype == "mxfp4":
        return 0.5 * width + width / 32.0
    raise ValueError(dtype)


def kv_bytes(w, ctx):
    """KV bytes one decode step reads: every context row of every request
    and KV head, once."""
    return sum(ctx) * w.Hkv * kv_bytes_per_token(w.Dk, w.Dv, w.v_alias_k, w.dtype)


def attn_flops(w, ctx):
    """Flops of the two contractions: 2 G (Dk + Dv) per token and KV head."""
    return sum(ctx) * w.Hkv * w.G * 2.0 * (w.Dk + w.Dv)


def page_kv_read_us(batch, tokens, kv_heads, tp, head_dim, bytes_per_element, bw=HBM_PEAK_BYTES_PER_S):
    """KV-read time per layer of one GPU in a TP group of `tp` GPUs: each GPU
    reads ceil(kv_heads / tp) heads (at least one) of K and V."""
    heads = max(1, math.ceil(kv_heads / tp))
    return 2.0 * heads * head_dim * tokens * bytes_per_element * batch / bw * 1e6
