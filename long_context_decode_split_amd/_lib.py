"""ctypes loader for libhelixdecode.so and the C structs of helixdecode.h."""

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first, so the library binds to the same one)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhelixdecode.so")

HX_OK, HX_EINVAL, HX_EUNSUPPORTED, HX_EHIP, HX_ENOSPC = 0, 1, 2, 3, 4
HX_KV_BF16, HX_KV_FP8_E4M3, HX_KV_MXFP4 = 0, 1, 2
HX_FLAG_P_BF16 = 1
STATUS_NAMES = {0: "HX_OK", 1: "HX_EINVAL", 2: "HX_EUNSUPPORTED", 3: "HX_EHIP", 4: "HX_ENOSPC"}


class hx_kv_desc(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("v_alias_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("cap", ctypes.c_int64)]


class hx_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


class hx_kv_layout_info(ctypes.Structure):
    _fields_ = [("k_bytes", ctypes.c_size_t), ("v_bytes", ctypes.c_size_t), ("k_scale_bytes", ctypes.c_size_t),
                ("v_scale_bytes", ctypes.c_size_t), ("k_tile_bytes", ctypes.c_size_t),
                ("v_tile_bytes", ctypes.c_size_t), ("n_max", ctypes.c_int64)]


class hx_kv_pool(ctypes.Structure):
    _fields_ = [("planes", hx_kv_cache), ("block_table", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


P_DESC = ctypes.POINTER(hx_kv_desc)
P_POOL = ctypes.POINTER(hx_kv_pool)
P_CACHE = ctypes.POINTER(hx_kv_cache)
VP = ctypes.c_void_p
I32, I64, F32, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
P_I64 = ctypes.POINTER(ctypes.c_int64)
P_I32 = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); every symbol include/helixdecode.h declares
SIGNATURES = {
    "hx_last_error": (ctypes.c_char_p, []),
    "hx_version": (ctypes.c_char_p, []),
    "hx_kv_layout": (I32, [P_DESC, ctypes.POINTER(hx_kv_layout_info)]),
    "hx_slot": (I32, [I64, I32, P_I32, P_I64]),
    "hx_slice_len": (I32, [I64, I32, I32, P_I64]),
    "hx_kv_tile_offset": (I32, [P_DESC, I32, I32, I32, P_I64]),
    "hx_kv_append": (I32, [P_DESC, P_CACHE, VP, VP, VP, VP, P_I64, P_I32, I32, VP]),
    "hx_kv_append_bf16": (I32, [P_DESC, P_CACHE, VP, VP, P_I64, P_I32, I32, VP]),
    "hx_kv_dequant": (I32, [P_DESC, P_CACHE, I32, I32, I32, I64, I64, VP, VP, VP]),
    "hx_workspace_size": (I32, [P_DESC, I32, ctypes.POINTER(SZ)]),
    "hx_workspace_init": (I32, [VP, SZ, VP]),
    "hx_decode_attn_partial": (I32, [P_DESC, P_CACHE, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_attn": (I32, [P_DESC, P_CACHE, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_attn_noalloc": (I32, [P_DESC, P_CACHE, VP, I32, P_I64, F32, VP, VP, VP]),
    "hx_lse_combine": (I32, [I32, I32, I32, I32, VP, VP, VP, VP, VP]),
    "hx_pool_layout": (I32, [P_DESC, I32, ctypes.POINTER(hx_kv_layout_info)]),
    "hx_kv_append_paged": (I32, [P_DESC, P_POOL, VP, VP, VP, VP, P_I64, P_I32, I32, VP]),
    "hx_kv_append_bf16_paged": (I32, [P_DESC, P_POOL, VP, VP, P_I64, P_I32, I32, VP]),
    "hx_kv_dequant_paged": (I32, [P_DESC, P_POOL, I32, I32, I32, I64, I64, VP, VP, VP]),
    "hx_decode_attn_partial_paged": (I32, [P_DESC, P_POOL, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_attn_paged": (I32, [P_DESC, P_POOL, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_step": (I32, [P_DESC, P_CACHE, VP, VP, VP, VP, I32, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_step_paged": (I32, [P_DESC, P_POOL, VP, VP, VP, VP, I32, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_step_bf16": (I32, [P_DESC, P_CACHE, VP, VP, I32, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_decode_step_bf16_paged": (I32, [P_DESC, P_POOL, VP, VP, I32, VP, I32, P_I64, F32, VP, VP, VP, SZ, VP]),
    "hx_block_pool_create": (I32, [I32, ctypes.POINTER(VP)]),
    "hx_block_pool_destroy": (None, [VP]),
    "hx_block_pool_free_count": (I32, [VP, P_I32]),
    "hx_block_pool_reserve": (I32, [VP, P_DESC, P_I32, I32, I64, P_I32]),
    "hx_block_pool_release": (I32, [VP, P_DESC, P_I32, I32]),
    "hx_trace_begin": (I32, [I32, VP]),
    "hx_trace_mark": (I32, [ctypes.c_char_p, VP]),
    "hx_trace_end": (I32, [P_I32, ctypes.POINTER(F32), ctypes.c_char_p]),
    "hx_read_probe": (I32, [VP, I64, VP, VP]),
}

HX_READ_PROBE_BLOCKS = 1024

_lib = None


class HXError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded library (loaded once).  Raises if it has not been built:
    there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_decode_split_amd.build` "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status):
    if status != HX_OK:
        raise HXError(status, lib().hx_last_error().decode())
