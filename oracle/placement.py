"""KV placement over KV-parallel slices (oracle; test infrastructure only).

Definition followed
-------------------
"Helix Parallelism" summary (fdeinterviews.com), paragraph on Helix's two
layouts: new KV entries rotate across the KV-parallel ranks every 16 tokens.
NVIDIA technical blog (open-lab.net, Korean), section on distributed KV
placement: with two ranks, tokens 1-16 land on rank 0 and tokens 17-32 on
rank 1.

Reading: tokens are counted from 0 per request, so token t belongs to the
16-token group t // 16, and groups are dealt to the P slices in turn,
starting at slice 0.  Inside a slice, rows keep arrival order.  The page's
1-based "1-16" is our 0..15.

This module enumerates; it does not reuse any closed form from the library.
"""

CHUNK = 16


def slot(t: int, P: int):
    """Slice and local row of token ``t`` (0-based) among ``P`` slices.

    Group g = t // 16 goes to slice g mod P; it is that slice's
    (g // P)-th group, so the local row is (g // P) * 16 + t mod 16.
    """
    if t < 0 or P < 1:
        raise ValueError("t must be >= 0 and P >= 1")
    g = t // CHUNK
    return g % P, (g // P) * CHUNK + t % CHUNK


def slice_tokens(n: int, P: int, r: int):
    """Token indices held by slice ``r`` when the request has ``n`` tokens,
    listed in local-row order (found by enumerating every token)."""
    rows = {}
    for t in range(n):
        rr, j = slot(t, P)
        if rr == r:
            rows[j] = t
    # local rows of a slice must be 0..L-1 with no gap
    assert sorted(rows) == list(range(len(rows)))
    return [rows[j] for j in range(len(rows))]


def slice_len(n: int, P: int, r: int) -> int:
    """Number of rows slice ``r`` holds for an ``n``-token request.

    Written as full rounds of P groups plus the share of the last, partial
    round: the partial round deals its leftover tokens to slices 0, 1, ...
    in 16-token pieces.
    """
    round_tokens = CHUNK * P
    full_rounds = n // round_tokens
    left = n - full_rounds * round_tokens
    mine = left - CHUNK * r
    mine = 0 if mine < 0 else (CHUNK if mine > CHUNK else mine)
    return full_rounds * CHUNK + mine


# ---------------------------------------------------------------------------
# Block-pool (paged) storage of the same placement.
#
# The pages fix where a token goes (slice, arrival order) but not how a
# slice's rows are stored.  A serving cache that grows per request keeps each
# slice as a list of 16-row blocks taken from a shared pool (the 16-token
# group is the placement unit: Helix summary, paragraph on Helix's two
# layouts; the stated goal of the rotation is an even memory fill).  Reading:
# local row j of slice r of request b lives in block table[b][r][j // 16],
# row j % 16 of that block.


def blocks_needed(n: int, P: int, r: int) -> int:
    """Blocks slice ``r`` occupies when the request has ``n`` tokens: the
    distinct 16-row groups among its rows (found by enumeration)."""
    return len({j // CHUNK for j in (slot(t, P)[1] for t in range(n) if slot(t, P)[0] == r)})


def block_row(t: int, P: int, table_b):
    """(block id, row inside the block) of token ``t`` of a request whose
    per-slice block lists are ``table_b[r][c]``."""
    r, j = slot(t, P)
    return table_b[r][j // CHUNK], j % CHUNK
