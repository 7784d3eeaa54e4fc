"""Thin Python binding of the helixdecode C ABI (include/helixdecode.h).

Every function here only turns torch tensors into pointers and host arrays
into ctypes arrays, then calls the library entry point of the same name; all
device work runs in the library's HIP kernels.  Errors raise ``HXError``.
PyTorch provides device memory and the current stream, nothing else.
"""

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from ._lib import (HX_FLAG_P_BF16, HX_KV_BF16, HX_KV_FP8_E4M3, HX_KV_MXFP4, HXError, check, hx_kv_cache,
                   hx_kv_desc, hx_kv_layout_info, hx_kv_pool, lib)

__all__ = ["HXError", "HX_FLAG_P_BF16", "KVDesc", "KVCache", "KVPool", "DTYPES", "kv_layout", "pool_layout", "slot", "slice_len",
           "kv_tile_offset", "kv_append", "kv_append_bf16", "kv_dequant", "kv_append_paged", "kv_append_bf16_paged",
           "kv_dequant_paged", "workspace_size", "workspace_init", "decode_attn_partial", "decode_attn",
           "decode_attn_noalloc", "decode_attn_partial_paged", "decode_attn_paged", "decode_step", "decode_step_paged", "decode_step_bf16", "decode_step_bf16_paged", "lse_combine",
           "version", "exported_symbols", "Trace"]

DTYPES = {"bf16": HX_KV_BF16, "fp8_e4m3": HX_KV_FP8_E4M3, "mxfp4": HX_KV_MXFP4}


@dataclass(frozen=True)
class KVDesc:
    """Mirror of ``hx_kv_desc``."""
    P: int
    B: int
    Hkv: int
    Dk: int
    Dv: int
    v_alias_k: bool
    dtype: str
    cap: int
    flags: int = 0      # HX_FLAG_P_BF16: MLA value product with P rounded once to bf16

    def c(self):
        return hx_kv_desc(self.P, self.B, self.Hkv, self.Dk, self.Dv, int(self.v_alias_k), DTYPES[self.dtype],
                          int(self.flags), self.cap)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _i64(values):
    values = [int(v) for v in values]
    return (ctypes.c_int64 * len(values))(*values)


def version():
    return lib().hx_version().decode()


def exported_symbols():
    from ._lib import SIGNATURES
    return sorted(SIGNATURES)


def kv_layout(desc: KVDesc):
    info = hx_kv_layout_info()
    check(lib().hx_kv_layout(ctypes.byref(desc.c()), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in hx_kv_layout_info._fields_}


def slot(t, P):
    r = ctypes.c_int32()
    j = ctypes.c_int64()
    check(lib().hx_slot(t, P, ctypes.byref(r), ctypes.byref(j)))
    return r.value, j.value


def slice_len(n, P, r):
    out = ctypes.c_int64()
    check(lib().hx_slice_len(n, P, r, ctypes.byref(out)))
    return out.value


def kv_tile_offset(desc: KVDesc, which, m, d):
    out = ctypes.c_int64()
    check(lib().hx_kv_tile_offset(ctypes.byref(desc.c()), which, m, d, ctypes.byref(out)))
    return out.value


class KVCache:
    """The cache planes of one layer, allocated with torch on ``device``
    using the sizes ``hx_kv_layout`` reports.  ``fill`` sets every byte (use
    0xFF to make unwritten rows NaN in every format)."""

    def __init__(self, desc: KVDesc, device="cuda", fill=None):
        self.desc = desc
        lay = kv_layout(desc)
        self.layout = lay

        def plane(nbytes):
            if nbytes == 0:
                return None
            t = torch.empty(nbytes, dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            return t

        self.k = plane(lay["k_bytes"])
        self.v = plane(lay["v_bytes"])
        self.k_scale = plane(lay["k_scale_bytes"])
        self.v_scale = plane(lay["v_scale_bytes"])
        # the C structs of this cache, built once (the planes never move)
        self._desc_ref = ctypes.byref(desc.c())
        self._c = hx_kv_cache(_ptr(self.k), _ptr(self.v), _ptr(self.k_scale), _ptr(self.v_scale))
        self._ref = ctypes.byref(self._c)

    def c(self):
        return self._c

    def nbytes(self):
        return sum(t.numel() for t in (self.k, self.v, self.k_scale, self.v_scale) if t is not None)


def pool_layout(desc: KVDesc, num_blocks):
    info = hx_kv_layout_info()
    check(lib().hx_pool_layout(ctypes.byref(desc.c()), int(num_blocks), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in hx_kv_layout_info._fields_}


class KVPool:
    """A block-pool cache of one layer: planes of ``num_blocks`` blocks
    (torch, sizes from ``hx_pool_layout``), the host block table (numpy int32
    [B, P, cap/16], -1 = no block) that the library's host allocator
    (``hx_block_pool_*``) edits, and its device copy ``table``, refreshed by
    ``sync()``.  ``desc.cap`` bounds the rows a slice can list."""

    def __init__(self, desc: KVDesc, num_blocks, device="cuda", fill=None):
        self.desc = desc
        self.num_blocks = int(num_blocks)
        self.layout = lay = pool_layout(desc, num_blocks)

        def plane(nbytes):
            if nbytes == 0:
                return None
            t = torch.empty(nbytes, dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            return t

        self.k = plane(lay["k_bytes"])
        self.v = plane(lay["v_bytes"])
        self.k_scale = plane(lay["k_scale_bytes"])
        self.v_scale = plane(lay["v_scale_bytes"])
        self.table_host = np.full((desc.B, desc.P, desc.cap // 16), -1, dtype=np.int32)
        self.table = torch.full(self.table_host.shape, -1, dtype=torch.int32, device=device)
        handle = ctypes.c_void_p()
        check(lib().hx_block_pool_create(self.num_blocks, ctypes.byref(handle)))
        self._handle = handle

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h is not None and h.value:
            lib().hx_block_pool_destroy(h)
            self._handle = None

    def _table_ptr(self):
        return self.table_host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def reserve(self, b, n):
        """``hx_block_pool_reserve``: request b's lists cover n tokens; returns
        the number of blocks taken (host table only: call ``sync``)."""
        taken = ctypes.c_int32()
        check(lib().hx_block_pool_reserve(self._handle, ctypes.byref(self.desc.c()), self._table_ptr(), int(b), int(n),
                                          ctypes.byref(taken)))
        return taken.value

    def release(self, b):
        """``hx_block_pool_release``: every block of request b back to the pool."""
        check(lib().hx_block_pool_release(self._handle, ctypes.byref(self.desc.c()), self._table_ptr(), int(b)))

    def free_blocks(self):
        n = ctypes.c_int32()
        check(lib().hx_block_pool_free_count(self._handle, ctypes.byref(n)))
        return n.value

    def sync(self):
        """Copy the host table to the device table (ordered on the current stream)."""
        self.table.copy_(torch.from_numpy(self.table_host))

    def c(self):
        planes = hx_kv_cache(_ptr(self.k), _ptr(self.v), _ptr(self.k_scale), _ptr(self.v_scale))
        return hx_kv_pool(planes, _ptr(self.table), self.num_blocks, 0)

    def nbytes(self):
        return sum(t.numel() for t in (self.k, self.v, self.k_scale, self.v_scale) if t is not None)


def _count(count):
    return None if count is None else (ctypes.c_int32 * len(count))(*[int(c) for c in count])


def kv_append(cache: KVCache, k_new, v_new, k_scale_new, v_scale_new, pos, count=None, stream=None):
    """``hx_kv_append``: token-major storage-format tensors of shape
    [B, Hkv, n_new, ...]; ``pos`` (and ``count``) are host sequences of B ints."""
    n_new = k_new.shape[2]
    cnt = None if count is None else (ctypes.c_int32 * len(count))(*[int(c) for c in count])
    check(lib().hx_kv_append(cache._desc_ref, cache._ref, _ptr(k_new), _ptr(v_new),
                             _ptr(k_scale_new), _ptr(v_scale_new), _i64(pos), cnt, n_new, _stream(stream)))


def kv_append_bf16(cache: KVCache, k_new, v_new, pos, count=None, stream=None):
    """``hx_kv_append_bf16``: bf16 tensors [B, Hkv, n_new, D] quantised into
    the cache's storage format on the device; ``pos`` (and ``count``) are
    host sequences of B ints."""
    n_new = k_new.shape[2]
    cnt = None if count is None else (ctypes.c_int32 * len(count))(*[int(c) for c in count])
    check(lib().hx_kv_append_bf16(ctypes.byref(cache.desc.c()), ctypes.byref(cache.c()), _ptr(k_new), _ptr(v_new),
                                  _i64(pos), cnt, n_new, _stream(stream)))


def kv_dequant(cache: KVCache, r, b, g, j0, n, k_out, v_out=None, stream=None):
    check(lib().hx_kv_dequant(ctypes.byref(cache.desc.c()), ctypes.byref(cache.c()), r, b, g, j0, n, _ptr(k_out),
                              _ptr(v_out), _stream(stream)))


def kv_append_paged(pool: KVPool, k_new, v_new, k_scale_new, v_scale_new, pos, count=None, stream=None):
    """``hx_kv_append_paged``: ``kv_append`` into a block pool."""
    check(lib().hx_kv_append_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_scale_new), _ptr(v_scale_new), _i64(pos), _count(count), k_new.shape[2],
                                   _stream(stream)))


def kv_append_bf16_paged(pool: KVPool, k_new, v_new, pos, count=None, stream=None):
    """``hx_kv_append_bf16_paged``: ``kv_append_bf16`` into a block pool."""
    check(lib().hx_kv_append_bf16_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(k_new),
                                        _ptr(v_new), _i64(pos), _count(count), k_new.shape[2], _stream(stream)))


def kv_dequant_paged(pool: KVPool, r, b, g, j0, n, k_out, v_out=None, stream=None):
    check(lib().hx_kv_dequant_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), r, b, g, j0, n,
                                    _ptr(k_out), _ptr(v_out), _stream(stream)))


def workspace_size(desc: KVDesc, Hq):
    out = ctypes.c_size_t()
    check(lib().hx_workspace_size(ctypes.byref(desc.c()), Hq, ctypes.byref(out)))
    return out.value


def workspace_init(ws, stream=None):
    check(lib().hx_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def decode_attn_partial(cache: KVCache, q, ctx_len, scale, o_part, lse_part, ws, stream=None):
    """``hx_decode_attn_partial``: q bf16 [B, Hq, Dk] -> o_part f32
    [P, B, Hq, Dv], lse_part f32 [P, B, Hq]."""
    Hq = q.shape[1]
    check(lib().hx_decode_attn_partial(cache._desc_ref, cache._ref, _ptr(q), Hq,
                                       _i64(ctx_len), float(scale), _ptr(o_part), _ptr(lse_part), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))


def decode_attn(cache: KVCache, q, ctx_len, scale, o, lse, ws, stream=None):
    """``hx_decode_attn``: q bf16 [B, Hq, Dk] -> o f32 [B, Hq, Dv], lse f32
    [B, Hq] (the whole step).  ``ws`` is scratch of ``workspace_size`` bytes;
    it needs no initialisation."""
    Hq = q.shape[1]
    check(lib().hx_decode_attn(cache._desc_ref, cache._ref, _ptr(q), Hq, _i64(ctx_len),
                               float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)))


def decode_attn_noalloc(cache: KVCache, q, ctx_len, scale, o, lse, stream=None):
    """``hx_decode_attn_noalloc``: ``decode_attn`` on the library's fixed
    per-device scratch (no workspace argument; calls on one device must not
    overlap)."""
    check(lib().hx_decode_attn_noalloc(ctypes.byref(cache.desc.c()), ctypes.byref(cache.c()), _ptr(q), q.shape[1],
                                       _i64(ctx_len), float(scale), _ptr(o), _ptr(lse), _stream(stream)))


def decode_attn_partial_paged(pool: KVPool, q, ctx_len, scale, o_part, lse_part, ws, stream=None):
    """``hx_decode_attn_partial_paged``: ``decode_attn_partial`` on a block pool."""
    check(lib().hx_decode_attn_partial_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                             q.shape[1], _i64(ctx_len), float(scale), _ptr(o_part), _ptr(lse_part),
                                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def decode_attn_paged(pool: KVPool, q, ctx_len, scale, o, lse, ws, stream=None):
    """``hx_decode_attn_paged``: ``decode_attn`` on a block pool."""
    check(lib().hx_decode_attn_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(q), q.shape[1],
                                     _i64(ctx_len), float(scale), _ptr(o), _ptr(lse), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def decode_step(cache: KVCache, k_new, v_new, k_scale_new, v_scale_new, q, ctx_len, scale, o, lse, ws, stream=None):
    """``hx_decode_step``: append the newest ``k_new.shape[2]`` rows of every
    request (storage format, [B, Hkv, n_new, ...]) and attend: o f32
    [B, Hq, Dv], lse f32 [B, Hq]."""
    check(lib().hx_decode_step(cache._desc_ref, cache._ref, _ptr(k_new), _ptr(v_new),
                               _ptr(k_scale_new), _ptr(v_scale_new), k_new.shape[2], _ptr(q), q.shape[1],
                               _i64(ctx_len), float(scale), _ptr(o), _ptr(lse), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))


def decode_step_paged(pool: KVPool, k_new, v_new, k_scale_new, v_scale_new, q, ctx_len, scale, o, lse, ws,
                      stream=None):
    """``hx_decode_step_paged``: ``decode_step`` on a block pool."""
    check(lib().hx_decode_step_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(k_new), _ptr(v_new),
                                     _ptr(k_scale_new), _ptr(v_scale_new), k_new.shape[2], _ptr(q), q.shape[1],
                                     _i64(ctx_len), float(scale), _ptr(o), _ptr(lse), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def decode_step_bf16(cache: KVCache, k_new, v_new, q, ctx_len, scale, o, lse, ws, stream=None):
    """``hx_decode_step_bf16``: the newest ``k_new.shape[2]`` rows of every
    request as bf16 [B, Hkv, n_new, D], quantised into the cache's format
    inside the step, then attention: o f32 [B, Hq, Dv], lse f32 [B, Hq]."""
    check(lib().hx_decode_step_bf16(cache._desc_ref, cache._ref, _ptr(k_new), _ptr(v_new),
                                    k_new.shape[2], _ptr(q), q.shape[1], _i64(ctx_len), float(scale), _ptr(o),
                                    _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def decode_step_bf16_paged(pool: KVPool, k_new, v_new, q, ctx_len, scale, o, lse, ws, stream=None):
    """``hx_decode_step_bf16_paged``: ``decode_step_bf16`` on a block pool."""
    check(lib().hx_decode_step_bf16_paged(ctypes.byref(pool.desc.c()), ctypes.byref(pool.c()), _ptr(k_new),
                                          _ptr(v_new), k_new.shape[2], _ptr(q), q.shape[1], _i64(ctx_len),
                                          float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)))


def lse_combine(o_part, lse_part, o, lse, stream=None):
    """``hx_lse_combine``: o_part [P, B, Hq, Dv], lse_part [P, B, Hq] ->
    o [B, Hq, Dv], lse [B, Hq] (all float32)."""
    P, B, Hq, Dv = o_part.shape
    check(lib().hx_lse_combine(P, B, Hq, Dv, _ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), _stream(stream)))


class Trace:
    """``hx_trace_begin`` / ``hx_trace_end`` as a context manager: while it
    is open, every library launch is followed by a HIP event on its stream.
    ``launches`` then lists (kernel name, ms from the previous event to the
    end of that launch)."""

    NAME = 32

    def __init__(self, capacity=4096, stream=None):
        self.capacity = int(capacity)
        self.stream = stream
        self.launches = []

    def __enter__(self):
        check(lib().hx_trace_begin(self.capacity, _stream(self.stream)))
        return self

    def __exit__(self, *exc):
        n = ctypes.c_int32()
        ms = (ctypes.c_float * self.capacity)()
        names = ctypes.create_string_buffer(self.capacity * self.NAME)
        check(lib().hx_trace_end(ctypes.byref(n), ms, names))
        raw = names.raw
        self.launches = [(raw[i * self.NAME:(i + 1) * self.NAME].split(b"\0", 1)[0].decode(), float(ms[i]))
                         for i in range(n.value)]
        return False

    def mark(self, name, stream=None):
        """``hx_trace_mark``: an entry of the caller's own for the work it ran
        on the stream since the previous entry."""
        check(lib().hx_trace_mark(name.encode(), _stream(stream)))

    def by_kernel(self):
        """{kernel name: [ms of each launch]}"""
        out = {}
        for name, ms in self.launches:
            out.setdefault(name, []).append(ms)
        return out


def read_probe(src, out=None, stream=None):
    """``hx_read_probe``: one plain streaming read of the device tensor
    ``src`` (its bytes, a multiple of 16); returns ``out``, a uint32 tensor
    of ``HX_READ_PROBE_BLOCKS`` per-workgroup XORs of what was read."""
    from ._lib import HX_READ_PROBE_BLOCKS
    nbytes = src.numel() * src.element_size()
    if out is None:
        out = torch.empty(HX_READ_PROBE_BLOCKS, dtype=torch.int32, device=src.device)
    check(lib().hx_read_probe(src.data_ptr(), nbytes, out.data_ptr(), _stream(stream)))
    return out
