"""Host side of block-pool caches: the native block allocator
(hx_block_pool_*), plane sizes (hx_pool_layout) and the argument checks of
the paged entry points (all before any launch; no GPU needed).  Expected
block counts come from the oracle's enumeration (oracle/placement.py)."""

import ctypes

import numpy as np
import pytest

from long_context_decode_split_amd import api
from long_context_decode_split_amd._lib import (HX_EINVAL, HX_ENOSPC, HXError, hx_kv_cache, hx_kv_pool, lib)
from oracle import placement as opl
from tests import helpers as H


@pytest.fixture(scope="module", autouse=True)
def _built():
    H.ensure_built()


def _desc(P=4, B=3, cap=256, dtype="bf16", Hkv=2):
    return api.KVDesc(P=P, B=B, Hkv=Hkv, Dk=128, Dv=128, v_alias_k=False, dtype=dtype, cap=cap)


def _blocks(n, P):
    return sum(opl.blocks_needed(n, P, r) for r in range(P))


def test_pool_layout_sizes():
    for dtype, kt, st in (("bf16", 4096, 0), ("fp8_e4m3", 2048, 4)):
        lay = api.pool_layout(_desc(dtype=dtype), 37)
        assert lay["k_tile_bytes"] == kt and lay["k_bytes"] == 37 * 2 * kt and lay["v_bytes"] == 37 * 2 * kt
        assert lay["k_scale_bytes"] == 37 * 2 * st and lay["v_scale_bytes"] == 37 * 2 * st
        assert lay["n_max"] == 4 * 256
    lay = api.pool_layout(_desc(dtype="mxfp4"), 37)       # packed tiles: one plane
    assert lay["k_tile_bytes"] == 2176 and lay["k_bytes"] == 37 * 2 * 2176
    assert lay["v_bytes"] == lay["k_scale_bytes"] == lay["v_scale_bytes"] == 0
    mla = api.KVDesc(P=8, B=1, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="bf16", cap=64)
    lay = api.pool_layout(mla, 5)
    assert lay["k_bytes"] == 5 * 16 * 1152 and lay["v_bytes"] == 0
    with pytest.raises(HXError):
        api.pool_layout(_desc(), 0)


def test_reserve_grows_lists_by_the_placement():
    d = _desc()
    pool = api.KVPool(d, 200, device="cpu")
    seen = set()
    for b, steps in ((0, (1, 17, 64, 65, 300, 1000)), (2, (16, 129)), (1, (1023, 1024))):
        have = 0
        for n in steps:
            taken = pool.reserve(b, n)
            assert taken == _blocks(n, d.P) - _blocks(have, d.P)
            have = n
            for r in range(d.P):
                row = pool.table_host[b, r]
                k = opl.blocks_needed(n, d.P, r)
                assert np.all(row[:k] >= 0) and np.all(row[k:] == -1)
        ids = pool.table_host[b][pool.table_host[b] >= 0]
        assert len(set(ids.tolist())) == len(ids)
        assert not (seen & set(ids.tolist()))
        seen |= set(ids.tolist())
    assert pool.free_blocks() == 200 - len(seen)
    assert pool.reserve(0, 1000) == 0          # already covered: nothing taken, nothing moved
    before = pool.table_host.copy()
    assert pool.reserve(0, 10) == 0 and np.array_equal(before, pool.table_host)


def test_reserve_is_all_or_nothing_and_release_recycles():
    d = _desc(P=2, B=2, cap=128)
    pool = api.KVPool(d, 10, device="cpu")
    assert pool.reserve(0, 100) == _blocks(100, 2)        # 7 blocks
    snap = pool.table_host.copy()
    with pytest.raises(HXError) as e:
        pool.reserve(1, 100)                              # needs 7, 3 free
    assert e.value.status == HX_ENOSPC
    assert np.array_equal(snap, pool.table_host) and pool.free_blocks() == 3
    first = [int(x) for x in pool.table_host[0][pool.table_host[0] >= 0]]
    pool.release(0)
    assert np.all(pool.table_host[0] == -1) and pool.free_blocks() == 10
    assert pool.reserve(1, 100) == 7
    got = sorted(int(x) for x in pool.table_host[1][pool.table_host[1] >= 0])
    assert got == sorted(first)                           # the freed blocks come back first


def test_release_rejects_foreign_or_duplicate_entries():
    d = _desc(P=2, B=2, cap=128)
    pool = api.KVPool(d, 10, device="cpu")
    pool.reserve(0, 40)
    pool.reserve(1, 40)
    snap = pool.table_host.copy()
    # one block listed twice under request 0 (and also owned by request 1)
    pool.table_host[0, 0, 5] = int(snap[1, 0, 0])
    pool.table_host[0, 1, 6] = int(snap[1, 0, 0])
    with pytest.raises(HXError) as e:
        pool.release(0)
    assert e.value.status == HX_EINVAL
    pool.table_host[...] = snap
    pool.table_host[0, 1, 0] = int(snap[1, 1, 0])         # request 1's block, listed once under request 0
    with pytest.raises(HXError):
        pool.release(0)
    pool.table_host[...] = snap
    pool.table_host[0, 1, 6] = 12345
    with pytest.raises(HXError):
        pool.release(0)
    with pytest.raises(HXError):
        pool.reserve(0, 128)                              # an entry in range of the new rows is not a pool block
    pool.table_host[...] = snap
    assert pool.free_blocks() == 10 - 2 * _blocks(40, 2)
    pool.release(0)
    pool.release(1)
    assert pool.free_blocks() == 10


def test_reserve_rejects_a_block_listed_twice():
    """A request's own block listed under two of its entries: reserve refuses
    it (as release does), leaving the pool and the table unchanged, whether
    the duplicate lies inside the rows being covered or beyond them."""
    d = _desc(P=2, B=2, cap=128)
    pool = api.KVPool(d, 20, device="cpu")
    pool.reserve(0, 40)
    snap = pool.table_host.copy()
    free = pool.free_blocks()
    own = int(snap[0, 0, 0])
    for r, c in ((1, 1), (0, 6)):               # (1, 1) is needed for 100 tokens, (0, 6) is not
        pool.table_host[...] = snap
        pool.table_host[0, r, c] = own
        before = pool.table_host.copy()
        with pytest.raises(HXError) as e:
            pool.reserve(0, 100)
        assert e.value.status == HX_EINVAL and "twice" in str(e.value)
        assert np.array_equal(before, pool.table_host) and pool.free_blocks() == free
        with pytest.raises(HXError):
            pool.release(0)
    pool.table_host[...] = snap
    assert pool.reserve(0, 100) == _blocks(100, 2) - _blocks(40, 2)
    pool.release(0)
    assert pool.free_blocks() == 20


def test_allocator_argument_errors():
    L = lib()
    h = ctypes.c_void_p()
    assert L.hx_block_pool_create(0, ctypes.byref(h)) == HX_EINVAL
    assert L.hx_block_pool_create(4, None) == HX_EINVAL
    d = _desc(P=2, B=2, cap=64)
    pool = api.KVPool(d, 4, device="cpu")
    with pytest.raises(HXError):
        pool.reserve(2, 10)                               # request out of range
    with pytest.raises(HXError):
        pool.reserve(0, 2 * 64 + 1)                       # beyond P * cap
    with pytest.raises(HXError):
        pool.reserve(0, -1)
    assert L.hx_block_pool_free_count(None, None) == HX_EINVAL


def _fake_pool(desc, table=0x10000, num_blocks=8, reserved=0, scales=False):
    planes = hx_kv_cache(0x100000, 0x200000, 0x300000 if scales else None, 0x400000 if scales else None)
    return hx_kv_pool(planes, table, num_blocks, reserved)


@pytest.mark.parametrize("bad", ["null_table", "misaligned_table", "no_blocks", "reserved"])
def test_paged_calls_check_the_pool_before_launch(bad):
    d = _desc(P=2, B=1, cap=64)
    kw = {"null_table": dict(table=None), "misaligned_table": dict(table=0x10004), "no_blocks": dict(num_blocks=0),
          "reserved": dict(reserved=1)}[bad]
    pool = _fake_pool(d, **kw)
    L = lib()
    dc = ctypes.byref(d.c())
    pos = (ctypes.c_int64 * 1)(0)
    ctx = (ctypes.c_int64 * 1)(10)
    calls = [
        lambda: L.hx_kv_append_paged(dc, ctypes.byref(pool), 0x500000, 0x600000, None, None, pos, None, 1, None),
        lambda: L.hx_kv_append_bf16_paged(dc, ctypes.byref(pool), 0x500000, 0x600000, pos, None, 1, None),
        lambda: L.hx_kv_dequant_paged(dc, ctypes.byref(pool), 0, 0, 0, 0, 1, 0x700000, None, None),
        lambda: L.hx_decode_attn_partial_paged(dc, ctypes.byref(pool), 0x800000, 16, ctx, 0.1, 0x900000, 0xa00000,
                                               0xb00000, 1 << 30, None),
        lambda: L.hx_decode_attn_paged(dc, ctypes.byref(pool), 0x800000, 16, ctx, 0.1, 0x900000, 0xa00000,
                                       0xb00000, 1 << 30, None),
    ]
    for call in calls:
        assert call() == HX_EINVAL
        assert L.hx_last_error()
    assert L.hx_kv_append_paged(dc, None, 0x500000, 0x600000, None, None, pos, None, 1, None) == HX_EINVAL


def test_paged_calls_apply_the_dense_checks():
    d = _desc(P=2, B=1, cap=64)
    pool = _fake_pool(d)
    L = lib()
    dc = ctypes.byref(d.c())
    pos = (ctypes.c_int64 * 1)(2 * 64)                    # past P * cap
    assert L.hx_kv_append_paged(dc, ctypes.byref(pool), 0x500000, 0x600000, None, None, pos, None, 1, None) == HX_EINVAL
    ctx = (ctypes.c_int64 * 1)(0)                         # empty request
    assert L.hx_decode_attn_partial_paged(dc, ctypes.byref(pool), 0x800000, 16, ctx, 0.1, 0x900000, 0xa00000,
                                          0xb00000, 1 << 30, None) == HX_EINVAL
    assert L.hx_kv_dequant_paged(dc, ctypes.byref(pool), 2, 0, 0, 0, 1, 0x700000, None, None) == HX_EINVAL
