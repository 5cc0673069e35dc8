"""ctypes loader for libkvq.so (the C ABI declared in include/kvq.h)."""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t


class KvqCache(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("page_size", c_i32),
        ("num_pages", c_i32),
        ("num_slots", c_i32),
        ("had_block", c_i32),
        ("sink", c_i32),
        ("recent", c_i32),
        ("int4_pool", c_vp),
        ("int8_pool", c_vp),
        ("code_bits", c_i32),
        ("key_bits", c_i32 * 4),
    ]


# name -> (restype, argtypes); every symbol include/kvq.h declares
SIGNATURES = {
    "kvq_int4_pool_bytes": (c_sz, [ctypes.POINTER(KvqCache)]),
    "kvq_int8_pool_bytes": (c_sz, [ctypes.POINTER(KvqCache)]),
    "kv_quant_append": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_vp, c_vp, c_vp, c_i32,
                                c_vp, c_i32, c_vp, c_vp]),
    "kv_decode_attn_workspace_bytes": (c_sz, [ctypes.POINTER(KvqCache), c_i32, c_i32]),
    "kv_decode_attn": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_i32, c_vp, c_vp, c_i32,
                               c_vp, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "kv_decode_read_ceiling": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_i32, c_vp, c_vp, c_i32,
                                       c_vp, c_i32, c_vp, c_sz, c_vp]),
    "kv_decode_attn_noalloc": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_i32, c_vp, c_vp, c_i32,
                                       c_vp, c_i32, c_vp, c_vp, c_vp]),
    "kv_append_decode_attn": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                                      c_vp, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "kv_prefill_attn": (c_i32, [ctypes.POINTER(KvqCache), c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp,
                                c_i32, c_vp, c_vp, c_vp]),
    "kvq_status_string": (ctypes.c_char_p, [c_i32]),
    "kvq_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m decode_attention_int4_block_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class KvqError(RuntimeError):
    pass


def check(status: int, what: str) -> None:
    if status != 0:
        lib = load()
        msg = lib.kvq_status_string(status).decode()
        detail = lib.kvq_last_error().decode()
        raise KvqError(f"{what}: {msg} ({detail})")
