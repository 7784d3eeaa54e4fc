"""Softmax decode attention, per-slice partials and their combine (oracle;
test infrastructure only).  All arithmetic is fp64.

Definitions followed
--------------------
* Attention of one decode query over a request's history (the operation
  every KV slice performs on its part; Helix summary, paragraph on KV
  parallelism; ifai.io article, section "Decoupling attention and FFN",
  "local FlashAttention"): for query head h of KV group g and tokens t < n,
      s_t  = scale * sum_d q[h, d] * K[g, t, d]
      LSE  = ln sum_t exp(s_t)
      O    = sum_t exp(s_t - LSE) * V[g, t, :]
  The max score is subtracted before exp (an exact rewrite that only keeps
  exp in range).
* Per-slice partials (Helix summary, paragraph on KV parallelism): slice r
  applies the same definition to its own tokens only and returns its
  normalised output O_r and its LSE_r.  An empty slice returns O_r = 0,
  LSE_r = -inf (reading: it contributes weight exp(-inf) = 0).
* Combine (jaehun.me review, Prompt 1.3.2, boxed formula):
      O = sum_r O_r exp(LSE_r) / sum_r exp(LSE_r)
  and, for the combined log-sum-exp (reading: the log of the same
  denominator), LSE = ln sum_r exp(LSE_r).  Both are evaluated after
  multiplying numerator and denominator by exp(-max_r LSE_r).

GQA head mapping (reading): query head h uses KV head h // (Hq // Hkv).
"""

import numpy as np

CHUNK = 16
_BLOCK = 1 << 16  # tokens widened to fp64 at a time (memory only)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def attend(q, K, V, scale):
    """Unsplit attention of the query rows ``q [G, Dk]`` over ``K [n, Dk]``,
    ``V [n, Dv]``.  Returns ``(O [G, Dv], LSE [G])`` in fp64.

    Two passes over the tokens: all scores first (to find the global max),
    then the exponentials, their sum and the weighted sum of V.  K and V are
    widened to fp64 ``_BLOCK`` rows at a time; the softmax is never split.
    """
    q = _f64(q)
    G = q.shape[0]
    n = K.shape[0]
    Dv = V.shape[1]
    if n == 0:
        return np.zeros((G, Dv)), np.full(G, -np.inf)
    s = np.empty((n, G))
    for a in range(0, n, _BLOCK):
        s[a:a + _BLOCK] = (_f64(K[a:a + _BLOCK]) @ q.T) * scale
    m = s.max(axis=0)
    w = np.exp(s - m)
    denom = w.sum(axis=0)
    num = np.zeros((G, Dv))
    for a in range(0, n, _BLOCK):
        num += w[a:a + _BLOCK].T @ _f64(V[a:a + _BLOCK])
    return num / denom[:, None], m + np.log(denom)


def attend_heads(q, K, V, scale):
    """All query heads of one request.  ``q [Hq, Dk]``, ``K [Hkv, n, Dk]``,
    ``V [Hkv, n, Dv]`` -> ``(O [Hq, Dv], LSE [Hq])``."""
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    O = np.empty((Hq, V.shape[2]))
    L = np.empty(Hq)
    for g in range(Hkv):
        O[g * G:(g + 1) * G], L[g * G:(g + 1) * G] = attend(q[g * G:(g + 1) * G], K[g], V[g], scale)
    return O, L


def slice_mask(n, P, r):
    """Boolean mask over tokens 0..n-1 of those held by slice ``r``: token t
    belongs to the 16-token group t // 16, dealt to slice (t // 16) mod P."""
    t = np.arange(n)
    return (t // CHUNK) % P == r


def slice_partials(q, K, V, scale, P):
    """Per-slice partials of one KV group: ``(O_parts [P, G, Dv],
    LSE_parts [P, G])``; slice r attends over the tokens ``slice_mask``
    gives it (their order inside the slice does not change the result)."""
    n = K.shape[0]
    G = q.shape[0]
    O = np.empty((P, G, V.shape[1]))
    L = np.empty((P, G))
    for r in range(P):
        idx = np.nonzero(slice_mask(n, P, r))[0]
        O[r], L[r] = attend(q, K[idx], V[idx], scale)
    return O, L


def combine(O_parts, LSE_parts):
    """Combine partials along axis 0: ``O_parts [P, ..., Dv]``,
    ``LSE_parts [P, ...]`` -> ``(O [..., Dv], LSE [...])``.

    Where every part is empty (all LSE = -inf) the result is O = 0,
    LSE = -inf.
    """
    O_parts = _f64(O_parts)
    LSE_parts = _f64(LSE_parts)
    m = LSE_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(LSE_parts - m_safe)          # exp(-inf) = 0 for empty parts
    denom = w.sum(axis=0)
    num = (w[..., None] * O_parts).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(empty[..., None], 0.0, num / np.where(empty, 1.0, denom)[..., None])
        LSE = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, denom)))
    return O, LSE
