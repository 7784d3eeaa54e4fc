"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-only entry points and argument checks behave.

No test here launches device work on purpose; the one call that would launch
runs only when no GPU is present and must come back as HX_EHIP."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from long_context_decode_split_amd import _lib, api
from oracle import placement
from tests.helpers import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "helixdecode.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    ensure_built()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hx_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(_lib.SIGNATURES), (declared_symbols(), sorted(_lib.SIGNATURES))


def test_header_and_binding_constants_agree():
    """Every #define HX_... and enumerator of the header has the binding's value."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    consts = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(HX_[A-Z0-9_]+)\s+(\d+)\s*$", text, re.M)}
    consts.update({m.group(1): int(m.group(2)) for m in re.finditer(r"\b(HX_[A-Z0-9_]+)\s*=\s*(\d+)", text)})
    for name in ("HX_OK", "HX_EINVAL", "HX_EUNSUPPORTED", "HX_EHIP", "HX_ENOSPC", "HX_KV_BF16", "HX_KV_FP8_E4M3",
                 "HX_KV_MXFP4", "HX_FLAG_P_BF16", "HX_READ_PROBE_BLOCKS"):
        assert consts[name] == getattr(_lib, name), name


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\b(hx_[a-z_0-9]+)$", out, flags=re.M))
    missing = [s for s in declared_symbols() if s not in exported]
    assert not missing, missing
    lib = _lib.lib()
    for s in declared_symbols():
        assert getattr(lib, s) is not None


def test_version():
    assert "gfx950" in api.version()


def test_slot_matches_oracle():
    for P in (1, 2, 3, 4, 8, 13, 64):
        for t in list(range(0, 600)) + [2**20 - 1, 2**20, 2**31 + 7]:
            assert api.slot(t, P) == placement.slot(t, P), (t, P)


def test_slice_len_matches_oracle():
    for P in (1, 2, 4, 8, 13):
        for n in list(range(0, 400)) + [4096, 4137, 2**20, 2097152, 1234567]:
            for r in range(P):
                assert api.slice_len(n, P, r) == placement.slice_len(n, P, r)


def test_slot_errors():
    with pytest.raises(api.HXError) as e:
        api.slot(-1, 4)
    assert e.value.status == _lib.HX_EINVAL
    with pytest.raises(api.HXError):
        api.slot(3, 0)
    with pytest.raises(api.HXError):
        api.slice_len(5, 4, 4)


DESCS = [
    api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64),
    api.KVDesc(P=8, B=3, Hkv=2, Dk=128, Dv=128, v_alias_k=False, dtype="fp8_e4m3", cap=32),
    api.KVDesc(P=8, B=1, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="mxfp4", cap=48),
    api.KVDesc(P=2, B=1, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="bf16", cap=16),
    api.KVDesc(P=2, B=2, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="fp8_e4m3", cap=32),
    api.KVDesc(P=4, B=1, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="mxfp4", cap=16),
]


def _packed(desc):
    """One plane of packed tiles: GQA MXFP4, and quantised MLA latent rows."""
    return desc.dtype == "mxfp4" or (desc.v_alias_k and desc.dtype != "bf16")


@pytest.mark.parametrize("desc", DESCS, ids=lambda d: f"{d.dtype}-{d.Dk}")
def test_layout_sizes(desc):
    lay = api.kv_layout(desc)
    tiles = desc.P * desc.B * desc.Hkv * desc.cap // 16
    bits = {"bf16": 16, "fp8_e4m3": 8, "mxfp4": 4}[desc.dtype]
    codes = 16 * desc.Dk * bits // 8
    assert lay["n_max"] == desc.P * desc.cap
    if _packed(desc):
        # one plane: GQA MXFP4 tiles hold K codes, V codes, K e8m0, V e8m0; MLA
        # tiles the latent codes, then the fp32 group scale padded to 16 bytes
        # (fp8) or the rows' e8m0 bytes (MXFP4)
        want = {("mxfp4", 128): 2 * codes + 2 * 16 * desc.Dk // 32, ("fp8_e4m3", 576): codes + 16,
                ("mxfp4", 576): codes + 16 * desc.Dk // 32}[(desc.dtype, desc.Dk)]
        assert lay["k_tile_bytes"] == want in (2176, 9232, 4896)
        assert lay["k_bytes"] == tiles * want
        assert lay["v_bytes"] == lay["k_scale_bytes"] == lay["v_scale_bytes"] == lay["v_tile_bytes"] == 0
        return
    assert lay["k_tile_bytes"] == codes
    assert lay["k_bytes"] == tiles * lay["k_tile_bytes"]
    if desc.v_alias_k:
        assert lay["v_bytes"] == 0
    else:
        assert lay["v_bytes"] == tiles * 16 * desc.Dv * bits // 8
    scale = {"bf16": 0, "fp8_e4m3": 4}[desc.dtype]
    assert lay["k_scale_bytes"] == tiles * scale


@pytest.mark.parametrize("desc", DESCS, ids=lambda d: f"{d.dtype}-{d.Dk}")
def test_tile_layout_is_a_bijection(desc):
    """Every code element of K and V (and every MXFP4 scale byte of a packed
    tile) has its own place, and together they fill the tile exactly."""
    lay = api.kv_layout(desc)
    bits = {"bf16": 16, "fp8_e4m3": 8, "mxfp4": 4}[desc.dtype]
    unit = {16: 4, 8: 2, 4: 1}[bits]            # off2 units per element
    packed = _packed(desc)
    for which, width in ((0, desc.Dk), (1, desc.Dv)):
        if which == 1 and desc.v_alias_k:
            continue
        offs = set()
        for m in range(16):
            for d in range(width):
                o2 = api.kv_tile_offset(desc, which, m, d)
                assert o2 % unit == 0
                offs.add(o2 // unit)
        codes = 16 * width * bits // 8
        lo = codes * 8 // bits if packed and which == 1 else 0    # packed: V codes follow K codes
        assert offs == set(range(lo, lo + codes * 8 // bits)), "elements must fill their part of the tile once"
    if packed and desc.dtype == "fp8_e4m3":   # MLA: the group scale right after the codes, for every element
        assert {api.kv_tile_offset(desc, 2, m, d) for m in (0, 7, 15) for d in (0, 300, 575)} == {2 * 16 * desc.Dk}
    elif packed:
        scale_bytes = set()
        for which in ((2,) if desc.v_alias_k else (2, 3)):
            for m in range(16):
                for d in range(0, desc.Dk, 32):
                    o2 = api.kv_tile_offset(desc, which, m, d)
                    assert o2 % 2 == 0 and api.kv_tile_offset(desc, which, m, d + 31) == o2
                    scale_bytes.add(o2 // 2)
        first = 16 * desc.Dk // 2 * (1 if desc.v_alias_k else 2)
        assert scale_bytes == set(range(first, lay["k_tile_bytes"])), "the e8m0 bytes end the tile"


def test_gqa_bf16_tile_gives_lane_fragments():
    """Each 1 KiB of a K tile is one wave-wide 16-byte-per-lane load: lane
    16h+m holds token m, columns 32s+8h..+7 of step s."""
    desc = DESCS[0]
    for s in range(4):
        for lane in range(64):
            m, h = lane % 16, lane // 16
            for e in range(8):
                assert api.kv_tile_offset(desc, 0, m, 32 * s + 8 * h + e) // 2 == s * 1024 + lane * 16 + 2 * e


def test_tile_offset_errors():
    with pytest.raises(api.HXError):
        api.kv_tile_offset(DESCS[0], 0, 16, 0)
    with pytest.raises(api.HXError):
        api.kv_tile_offset(DESCS[0], 2, 0, 0)          # bf16: no scales
    with pytest.raises(api.HXError):
        api.kv_tile_offset(DESCS[2], 4, 0, 0)
    with pytest.raises(api.HXError):
        api.kv_tile_offset(DESCS[3], 1, 0, 0)          # MLA: V aliases K
    assert api.kv_tile_offset(DESCS[1], 3, 5, 77) == 0  # fp8: the tile's one float


@pytest.mark.parametrize("bad,status", [
    (dict(P=0), _lib.HX_EINVAL), (dict(P=65), _lib.HX_EINVAL), (dict(cap=40), _lib.HX_EINVAL),
    (dict(cap=0), _lib.HX_EINVAL), (dict(B=0), _lib.HX_EINVAL), (dict(Dk=64, Dv=64), _lib.HX_EUNSUPPORTED),
    (dict(flags=2), _lib.HX_EINVAL), (dict(flags=-1), _lib.HX_EINVAL),
    (dict(Dk=576, Dv=512, v_alias_k=False), _lib.HX_EUNSUPPORTED),
    (dict(Dk=576, Dv=256, v_alias_k=True, dtype="fp8_e4m3"), _lib.HX_EUNSUPPORTED),
])
def test_desc_errors(bad, status):
    base = dict(P=4, B=1, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    base.update(bad)
    with pytest.raises(api.HXError) as e:
        api.kv_layout(api.KVDesc(**base))
    assert e.value.status == status
    assert _lib.lib().hx_last_error().decode()


def test_workspace_size_and_heads():
    d = DESCS[0]
    assert api.workspace_size(d, 8) > 0
    for G in (17, 34, 64, 128):        # wide GQA groups
        assert api.workspace_size(api.KVDesc(**{**d.__dict__, "Hkv": 1}), G) > api.workspace_size(d, 8)
    with pytest.raises(api.HXError) as e:
        api.workspace_size(api.KVDesc(**{**d.__dict__, "Hkv": 1}), 129)   # G = 129 > 128
    assert e.value.status == _lib.HX_EUNSUPPORTED
    with pytest.raises(api.HXError) as e:
        api.workspace_size(DESCS[1], 3)   # not a multiple of Hkv = 2
    assert e.value.status == _lib.HX_EINVAL
    with pytest.raises(api.HXError) as e:
        api.workspace_size(DESCS[3], 64)   # MLA takes G = 128
    assert e.value.status == _lib.HX_EUNSUPPORTED


def _fake(addr):
    return ctypes.c_void_p(addr)


def _partial(desc, ctx, q=0x10000, ws=0x20000, ws_bytes=1 << 30, scale=0.1, Hq=8, o=0x30000, lse=0x40000,
             cache=None):
    L = _lib.lib()
    cache = cache or _lib.hx_kv_cache(0x50000, 0x60000, None, None)
    ctx_arr = (ctypes.c_int64 * len(ctx))(*ctx)
    return L.hx_decode_attn_partial(ctypes.byref(desc.c()), ctypes.byref(cache), _fake(q), Hq, ctx_arr,
                                    ctypes.c_float(scale), _fake(o), _fake(lse), _fake(ws), ws_bytes, None)


def test_partial_argument_checks_return_before_launch():
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    assert _partial(d, [0, 5]) == _lib.HX_EINVAL            # empty context
    assert _partial(d, [5, 4 * 64 + 1]) == _lib.HX_EINVAL   # beyond P * cap
    assert _partial(d, [5, 5], q=0x10008) == _lib.HX_EINVAL  # misaligned
    assert _partial(d, [5, 5], ws_bytes=16) == _lib.HX_EINVAL  # workspace too small
    assert _partial(d, [5, 5], scale=0.0) == _lib.HX_EINVAL
    assert _partial(d, [5, 5], scale=float("nan")) == _lib.HX_EINVAL
    assert _partial(d, [5, 5], Hq=0) == _lib.HX_EINVAL
    assert _partial(d, [5, 5], cache=_lib.hx_kv_cache(0x50000, None, None, None)) == _lib.HX_EINVAL


def test_decode_attn_argument_checks():
    L = _lib.lib()
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    cache = _lib.hx_kv_cache(0x50000, 0x60000, None, None)
    ctx = (ctypes.c_int64 * 2)(5, 17)

    def call(o=0x30000, lse=0x40000, ws_bytes=1 << 30):
        return L.hx_decode_attn(ctypes.byref(d.c()), ctypes.byref(cache), _fake(0x10000), 8, ctx, ctypes.c_float(0.1),
                                _fake(o) if o else None, _fake(lse) if lse else None, _fake(0x20000), ws_bytes, None)

    assert call(o=0) == _lib.HX_EINVAL
    assert call(lse=0) == _lib.HX_EINVAL
    assert call(o=0x30004) == _lib.HX_EINVAL     # misaligned
    assert call(ws_bytes=16) == _lib.HX_EINVAL
    if not torch.cuda.is_available():
        assert call() == _lib.HX_EHIP             # valid arguments reach the launch


def test_decode_step_argument_checks():
    L = _lib.lib()
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    cache = _lib.hx_kv_cache(0x50000, 0x60000, None, None)

    def call(ctx=(5, 17), n_new=1, o=0x30000, kn=0x70000, vn=0x80000, ks=None):
        c = (ctypes.c_int64 * 2)(*ctx)
        return L.hx_decode_step(ctypes.byref(d.c()), ctypes.byref(cache), _fake(kn) if kn else None,
                                _fake(vn) if vn else None, _fake(ks) if ks else None, None, n_new, _fake(0x10000), 8,
                                c, ctypes.c_float(0.1), _fake(o) if o else None, _fake(0x40000), _fake(0x20000),
                                1 << 30, None)

    assert call(ctx=(5, 1), n_new=2) == _lib.HX_EINVAL     # a request shorter than its new rows
    assert call(n_new=0) == _lib.HX_EINVAL
    assert call(o=0) == _lib.HX_EINVAL
    assert call(vn=0) == _lib.HX_EINVAL                    # V rows missing
    assert call(ks=0x90000) == _lib.HX_EINVAL              # bf16 caches take no scales
    assert call(kn=0x70004) == _lib.HX_EINVAL              # misaligned
    assert call(ctx=(5, 4 * 64 + 1)) == _lib.HX_EINVAL     # beyond P * cap
    if not torch.cuda.is_available():
        assert call() == _lib.HX_EHIP


def test_decode_attn_noalloc_argument_checks():
    """The fixed-scratch entry point checks its arguments, and whether its
    split records and slice partials fit the library's 128 MiB scratch,
    before it touches the device."""
    L = _lib.lib()

    def call(d, cache, ctx, Hq, o=0x30000, lse=0x40000, q=0x10000):
        c = (ctypes.c_int64 * len(ctx))(*ctx)
        return L.hx_decode_attn_noalloc(ctypes.byref(d.c()), ctypes.byref(cache), _fake(q), Hq, c, ctypes.c_float(0.1),
                                        _fake(o) if o else None, _fake(lse), None)

    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    cache = _lib.hx_kv_cache(0x50000, 0x60000, None, None)
    assert call(d, cache, (5, 17), 8, o=0) == _lib.HX_EINVAL
    assert call(d, cache, (5, 17), 8, lse=0x40004) == _lib.HX_EINVAL      # misaligned
    assert call(d, cache, (5, 0), 8) == _lib.HX_EINVAL                      # empty request
    assert call(d, cache, (5, 17), 0) == _lib.HX_EINVAL                     # no query heads
    # 64 requests x 128 MLA heads x 64 slices: slice partials alone are 1 GiB
    big = api.KVDesc(P=64, B=64, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype="bf16", cap=16)
    rc = call(big, _lib.hx_kv_cache(0x50000, None, None, None), [100] * 64, 128)
    assert rc == _lib.HX_EINVAL and b"fixed" in L.hx_last_error()
    if not torch.cuda.is_available():
        assert call(d, cache, (5, 17), 8) == _lib.HX_EHIP                   # valid arguments reach the device


def test_trace_argument_checks():
    L = _lib.lib()
    n = ctypes.c_int32()
    ms = (ctypes.c_float * 4)()
    names = ctypes.create_string_buffer(4 * 32)
    assert L.hx_trace_end(ctypes.byref(n), ms, names) == _lib.HX_EINVAL        # none open
    assert L.hx_trace_mark(b"x", None) == _lib.HX_EINVAL                        # none open
    assert L.hx_trace_begin(0, None) == _lib.HX_EINVAL
    assert L.hx_trace_begin(1 << 21, None) == _lib.HX_EINVAL
    if not torch.cuda.is_available():
        assert L.hx_trace_begin(4, None) == _lib.HX_EHIP                       # events need a device


def test_read_probe_argument_checks():
    L = _lib.lib()
    out = 0x80000
    assert L.hx_read_probe(None, 1024, out, None) == _lib.HX_EINVAL
    assert L.hx_read_probe(0x40000, 1024, None, None) == _lib.HX_EINVAL
    assert L.hx_read_probe(0x40008, 1024, out, None) == _lib.HX_EINVAL      # misaligned
    assert L.hx_read_probe(0x40000, 0, out, None) == _lib.HX_EINVAL
    assert L.hx_read_probe(0x40000, 1000, out, None) == _lib.HX_EINVAL      # not a multiple of 16
    if not torch.cuda.is_available():
        assert L.hx_read_probe(0x40000, 1024, out, None) == _lib.HX_EHIP    # valid arguments reach the launch


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_partial_without_device_is_hx_ehip():
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    assert _partial(d, [5, 17]) == _lib.HX_EHIP


def test_append_argument_checks():
    L = _lib.lib()
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="bf16", cap=64)
    cache = _lib.hx_kv_cache(0x50000, 0x60000, None, None)

    def call(pos, count=None, n_new=4, k=0x10000, v=0x20000, ks=None):
        pa = (ctypes.c_int64 * 2)(*pos)
        ca = None if count is None else (ctypes.c_int32 * 2)(*count)
        return L.hx_kv_append(ctypes.byref(d.c()), ctypes.byref(cache), _fake(k), _fake(v), ks, None, pa, ca, n_new,
                              None)

    assert call([0, 254]) == _lib.HX_EINVAL            # 254 + 4 > P * cap = 256
    assert call([-1, 0]) == _lib.HX_EINVAL
    assert call([0, 0], n_new=0) == _lib.HX_EINVAL
    assert call([0, 0], count=[5, 1]) == _lib.HX_EINVAL   # count > n_new
    assert call([0, 0], count=[-1, 1]) == _lib.HX_EINVAL
    assert call([0, 0], k=0x10002) == _lib.HX_EINVAL      # misaligned
    assert call([0, 0], v=0) == _lib.HX_EINVAL
    assert call([0, 0], ks=_fake(0x70000)) == _lib.HX_EINVAL   # bf16 takes no scales


def test_quantising_append_argument_checks():
    L = _lib.lib()
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=128, Dv=128, v_alias_k=False, dtype="fp8_e4m3", cap=64)
    cache = _lib.hx_kv_cache(0x50000, 0x60000, 0x70000, 0x80000)

    def call(pos, count=None, n_new=4, k=0x10000, v=0x20000, c=cache):
        pa = (ctypes.c_int64 * 2)(*pos)
        ca = None if count is None else (ctypes.c_int32 * 2)(*count)
        return L.hx_kv_append_bf16(ctypes.byref(d.c()), ctypes.byref(c), _fake(k), _fake(v), pa, ca, n_new, None)

    assert call([0, 254]) == _lib.HX_EINVAL            # 254 + 4 > P * cap = 256
    assert call([-1, 0]) == _lib.HX_EINVAL
    assert call([0, 0], n_new=0) == _lib.HX_EINVAL
    assert call([0, 0], count=[5, 1]) == _lib.HX_EINVAL   # count > n_new
    assert call([0, 0], k=0x10002) == _lib.HX_EINVAL      # misaligned
    assert call([0, 0], v=0) == _lib.HX_EINVAL
    assert call([0, 0], c=_lib.hx_kv_cache(0x50000, 0x60000, None, 0x80000)) == _lib.HX_EINVAL   # no K scales
    if not torch.cuda.is_available():
        assert call([0, 0]) == _lib.HX_EHIP               # valid arguments reach the launch


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "mxfp4"])
def test_quantised_mla_cache_argument_checks(dtype):
    """Quantised MLA caches: one packed plane (k), latent rows only (no V
    input), for the quantising and the storage-format appends and the step."""
    L = _lib.lib()
    d = api.KVDesc(P=4, B=2, Hkv=1, Dk=576, Dv=512, v_alias_k=True, dtype=dtype, cap=64)
    one = _lib.hx_kv_cache(0x50000, None, None, None)
    pa = (ctypes.c_int64 * 2)(0, 0)

    def bf16(k=0x10000, v=None, c=one):
        return L.hx_kv_append_bf16(ctypes.byref(d.c()), ctypes.byref(c), _fake(k), _fake(v), pa, None, 4, None)

    assert bf16(v=0x20000) == _lib.HX_EINVAL                               # V aliases K: no v_new
    assert bf16(k=0) == _lib.HX_EINVAL
    assert bf16(c=_lib.hx_kv_cache(0x50000, None, 0x70000, None)) == _lib.HX_EINVAL   # packed: one plane
    assert bf16(c=_lib.hx_kv_cache(0x50000, 0x60000, None, None)) == _lib.HX_EINVAL
    assert L.hx_kv_append(ctypes.byref(d.c()), ctypes.byref(one), _fake(0x10000), _fake(0x20000), _fake(0x30000),
                          None, pa, None, 4, None) == _lib.HX_EINVAL        # storage format: no v_new either
    assert L.hx_kv_append(ctypes.byref(d.c()), ctypes.byref(one), _fake(0x10000), None, None, None, pa, None, 4,
                          None) == _lib.HX_EINVAL                           # scales are required
    if not torch.cuda.is_available():
        assert bf16() == _lib.HX_EHIP                                      # valid arguments reach the launch


def test_dequant_and_combine_argument_checks():
    L = _lib.lib()
    d = DESCS[0]
    cache = _lib.hx_kv_cache(0x50000, 0x60000, None, None)
    assert L.hx_kv_dequant(ctypes.byref(d.c()), ctypes.byref(cache), 4, 0, 0, 0, 1, _fake(0x1000), None,
                           None) == _lib.HX_EINVAL
    assert L.hx_kv_dequant(ctypes.byref(d.c()), ctypes.byref(cache), 0, 0, 0, 60, 8, _fake(0x1000), None,
                           None) == _lib.HX_EINVAL
    assert L.hx_lse_combine(0, 1, 1, 1, _fake(16), _fake(32), _fake(48), _fake(64), None) == _lib.HX_EINVAL
    assert L.hx_lse_combine(2, 1, 1, 1, _fake(16), _fake(33), _fake(48), _fake(64), None) == _lib.HX_EINVAL
    assert L.hx_lse_combine(2, 1, 1, 1, None, _fake(32), _fake(48), _fake(64), None) == _lib.HX_EINVAL


C_CALLER = r"""
#include <stdio.h>
#include "helixdecode.h"

int main(void) {
  int32_t r; int64_t j, len;
  hx_kv_desc d = {8, 2, 1, 128, 128, 0, HX_KV_MXFP4, 0, 1024};
  hx_kv_layout_info lay;
  if (hx_slot(40, 2, &r, &j) != HX_OK) return 1;
  if (hx_slice_len(4137, 8, 2, &len) != HX_OK) return 2;
  if (hx_kv_layout(&d, &lay) != HX_OK) return 3;
  if (hx_slot(-1, 2, &r, &j) != HX_EINVAL || hx_last_error()[0] == 0) return 4;
  printf("%d %lld %lld %zu %zu\n", r, (long long)j, (long long)len, lay.k_bytes, lay.v_bytes);
  return 0;
}
"""


def test_header_is_plain_c(tmp_path):
    """A C99 program includes the header, links the library and calls its
    host-only entry points: the boundary needs no C++ and no torch."""
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe),
           f"-L{libdir}", "-lhelixdecode", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split()
    # token 40 with P = 2: group 2 -> slice 0, local row 16 + 8; slice 2 of a 4137-token request (P = 8): 521 rows
    assert out[:3] == ["0", "24", str(placement.slice_len(4137, 8, 2))]
    assert int(out[3]) == 8 * 2 * 1 * (1024 // 16) * 2176 and out[4] == "0"
