"""Decoders for the KV storage formats (oracle; test infrastructure only).

The pages say only that the KV cache is kept in FP4 (Helix summary,
paragraph on the TP roofline; Helix review, Prompt 1.1.1 hardware context)
and that the LSE rescale stays exact at FP4/FP8 (Helix review, Prompt 1.3.2,
"Numerical Stability").  They fix no format, so the cache formats are read as
the public OCP ones:

* fp8 "e4m3" (OCP 8-bit floating point, E4M3 variant): 1 sign, 4 exponent
  bits with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111
  is NaN, largest finite 448.
* e2m1 (OCP Microscaling MX v1.0, FP4 element): 1 sign, 2 exponent bits with
  bias 1, 1 mantissa bit, subnormal when the exponent field is 0.
* e8m0 (OCP MX v1.0 shared block scale): 2**(E-127), E = 255 is NaN.

Every value is built from the bit fields in fp64; no library cast is used.

Cache-level conventions (readings, since the pages are silent):

* fp8 cache: one fp32 scale per 16-token group of a (request, KV head,
  K or V); the dequantised value is the fp32 product code*scale rounded to
  nearest-even.
* MXFP4 cache: 32 consecutive elements of one token row share an e8m0
  scale; two e2m1 codes per byte, the even element in the low nibble.  The
  value code * 2**(E-127) is exact in fp64.
"""

import numpy as np


def fp8_e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


FP8_E4M3 = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

CHUNK = 16
MX_BLOCK = 32


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64; bf16 is the top half of fp32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_fp8(codes, scales):
    """fp8 e4m3 codes ``[..., n, D]`` (uint8) with one fp32 scale per
    16-token group ``[..., ceil(n/16)]`` -> float64 ``[..., n, D]``.

    Token t uses scale t // 16.  The value is fp32(code) * fp32(scale)
    rounded to fp32 (the product of two fp32 numbers rounded once), then
    widened.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32)
    n = codes.shape[-2]
    tok_scale = np.repeat(scales, CHUNK, axis=-1)[..., :n]
    vals = FP8_E4M3[codes].astype(np.float32)  # exact: e4m3 fits in fp32
    prod = vals * tok_scale[..., None]          # fp32 x fp32, one rounding
    return prod.astype(np.float64)


def dequant_mxfp4(packed, e8m0):
    """MXFP4 rows: ``packed [..., n, D/2]`` uint8 (even element in the low
    nibble) and ``e8m0 [..., n, D/32]`` uint8 -> float64 ``[..., n, D]``."""
    packed = np.asarray(packed, dtype=np.uint8)
    e8m0 = np.asarray(e8m0, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    vals = E2M1[codes]
    scale = np.repeat(E8M0[e8m0], MX_BLOCK, axis=-1)
    return vals * scale
