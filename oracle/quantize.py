"""Encoders for the KV storage formats, and the quantising append of new
bf16 rows into a cache chunk (oracle; test infrastructure only).

The pages fix neither the cache formats nor how new tokens are quantised;
they say the KV cache is kept in FP4 (Helix summary, paragraph on the TP
roofline) and that new KV is written round-robin as it is produced (Helix
summary, paragraph on Helix's two layouts).  The formats are the public OCP
ones (see oracle.codecs); the quantisation rules are these readings:

* fp8 e4m3 chunk (16 rows of one request, KV head, K or V): scale =
  amax / 448 in fp32 (1 when amax = 0); code = e4m3 nearest to the fp32
  quotient x / scale, ties to the even code, after clamping to [-448, 448].
* MXFP4 row block (32 consecutive elements of one row): E = clamp(floor(
  log2 amax) - 2, -127, 127) + 127; code = e2m1 nearest to x / 2^(E-127),
  ties to the even code, saturating at 6; a value that rounds to zero gets
  the positive zero code.
* Open-chunk policy for fp8 (rows of one chunk arriving over several
  appends): the stored scale only grows.  With m_old = 448 * scale_old when
  some stored code of the chunk is non-zero (else 0) and a = amax of the new
  rows: if a <= m_old the scale stays; otherwise it becomes a / 448 and the
  stored codes are re-encoded from their decoded values times
  scale_old / scale_new (fp32 quotient, fp32 product).  New rows are then
  encoded with the chunk's scale.  Appending a whole chunk at once is thus
  exactly the per-chunk rule above, and the scale always equals the chunk's
  running amax / 448.

Encoding is a nearest search over the value tables of oracle.codecs (fp64),
so no bit-level rounding trick is involved.
"""

import numpy as np

from oracle.codecs import E2M1, FP8_E4M3

CHUNK = 16
MX_BLOCK = 32
FP8_MAX = 448.0

# non-negative finite e4m3 values in code order (codes 0x00 .. 0x7E, increasing)
_E4M3_POS = FP8_E4M3[:0x7F]
# non-negative e2m1 values, codes 0 .. 7 (increasing)
_E2M1_POS = E2M1[:8]


def _nearest_even(table, a):
    """Index of the entry of the increasing `table` nearest to each a >= 0
    (a within the table's range); ties go to the even index."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = np.abs(a - table[lo])
    dhi = np.abs(table[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def encode_e4m3(x):
    """fp32 values already within [-448, 448] -> e4m3 codes (uint8), nearest
    with ties to the even code; the sign bit follows the sign of x
    (negative zero included)."""
    x = np.asarray(x, dtype=np.float32)
    idx = _nearest_even(_E4M3_POS, np.abs(x).astype(np.float64))
    return (idx | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def encode_e2m1(y):
    """fp32 values -> e2m1 codes (0..15), nearest with ties to the even code,
    magnitudes above 6 saturating to 6; zero magnitude gets code 0."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 6.0)
    idx = _nearest_even(_E2M1_POS, a)
    neg = (y < 0) & (idx > 0)
    return (idx | (neg.astype(np.int64) << 3)).astype(np.uint8)


def fp8_chunk_scale(amax):
    """Per-chunk scale: fp32 amax / 448, or 1 for an all-zero chunk."""
    a = np.float32(amax)
    return np.float32(a / np.float32(FP8_MAX)) if a > 0 else np.float32(1.0)


def quantize_fp8_rows(x, scale):
    """fp32 rows -> e4m3 codes with the given fp32 scale (x / scale in fp32,
    clamped to +-448)."""
    q = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    return encode_e4m3(np.clip(q, -FP8_MAX, FP8_MAX))


def append_fp8_chunk(codes, scale, n_old, x_new):
    """The open-chunk policy.  `codes` [16, D] uint8 holds the chunk's stored
    codes (rows < n_old are valid), `scale` its stored fp32 scale, `x_new`
    [k, D] the new rows (fp32 holding bf16 values), appended at rows
    n_old .. n_old + k - 1.  Returns the chunk's new (codes, scale)."""
    codes = np.array(codes, dtype=np.uint8, copy=True)
    x_new = np.asarray(x_new, dtype=np.float32)
    k = x_new.shape[0]
    assert 0 <= n_old and n_old + k <= CHUNK and k >= 1
    a = np.float32(np.max(np.abs(x_new)))
    old = codes[:n_old]
    m_old = np.float32(np.float32(scale) * np.float32(FP8_MAX)) if n_old and np.any(old & 0x7F) else np.float32(0)
    if n_old == 0:
        new_scale = fp8_chunk_scale(a)
    elif a <= m_old:
        new_scale = np.float32(scale)
    elif a > 0:
        new_scale = np.float32(a / np.float32(FP8_MAX))
        if m_old > 0:
            r = np.float32(np.float32(scale) / new_scale)
            y = (FP8_E4M3[old].astype(np.float32) * r).astype(np.float32)
            codes[:n_old] = encode_e4m3(np.clip(y, -FP8_MAX, FP8_MAX))
    else:
        new_scale = np.float32(scale)
    codes[n_old:n_old + k] = quantize_fp8_rows(x_new, new_scale)
    return codes, new_scale


def mxfp4_block_exponent(amax):
    """e8m0 code of a 32-element block: clamp(floor(log2 amax) - 2, -127,
    127) + 127 (an all-zero block gets 0)."""
    a = np.asarray(amax, dtype=np.float64)
    # floor(log2 a) exactly: a = m * 2^ex with m in [0.5, 1)
    _, ex = np.frexp(a)
    e = np.where(a > 0, ex.astype(np.float64) - 1.0 - 2.0, -127.0)
    e = np.clip(e, -127.0, 127.0)
    return (e + 127.0).astype(np.uint8)


def quantize_mxfp4_rows(x):
    """fp32 rows [n, D] -> (packed codes [n, D/2] uint8 with the even element
    in the low nibble, e8m0 [n, D/32] uint8)."""
    x = np.asarray(x, dtype=np.float32)
    n, D = x.shape
    xb = x.reshape(n, D // MX_BLOCK, MX_BLOCK)
    E = mxfp4_block_exponent(np.max(np.abs(xb), axis=-1).astype(np.float64))
    # y = x / 2^(E-127): a power-of-two scaling, exact in fp64 and in fp32
    y = (xb.astype(np.float64) * np.exp2(127.0 - E.astype(np.float64))[..., None]).astype(np.float32)
    codes = encode_e2m1(y).reshape(n, D)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, E
