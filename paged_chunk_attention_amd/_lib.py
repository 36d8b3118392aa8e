"""ctypes declarations of the C ABI in include/oomb.h.

The shared library is loaded from this package's directory. There is no fallback:
if liboomb.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboomb.so")

OOMB_OK, OOMB_ERR_INVALID, OOMB_ERR_UNSUPPORTED, OOMB_ERR_HIP, OOMB_ERR_WORKSPACE = range(5)
OOMB_DTYPE_BF16, OOMB_DTYPE_FP32 = 0, 1

P_i32 = ctypes.POINTER(c_int32)


class OombPool(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("page_size", c_int32), ("head_dim", c_int32),
        ("num_q_heads", c_int32), ("num_kv_heads", c_int32), ("reserved", c_int32),
        ("num_pages", c_int64), ("num_grad_pages", c_int64),
        ("k_pool", c_void_p), ("v_pool", c_void_p), ("k_summary", c_void_p),
        ("dk_pool", c_void_p), ("dv_pool", c_void_p),
    ]


P_pool = ctypes.POINTER(OombPool)

# name -> (restype, argtypes); mirrors include/oomb.h one to one.
SIGNATURES = {
    "oomb_status_string": (c_char_p, [c_int]),
    "oomb_last_error": (c_char_p, []),
    "oomb_abi_version": (c_int, []),
    "oomb_kv_append": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_int64,
                               c_int32, c_int64, c_void_p]),
    "oomb_page_summarize": (c_int, [P_pool, c_void_p, c_int64, c_int64, c_int64, c_int64,
                                    c_void_p]),
    "oomb_select_workspace_bytes": (c_size_t, [P_pool, c_int32, c_int64]),
    "oomb_select_pages": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int32,
                                  c_int64, c_int32, c_void_p, c_int64, c_void_p, c_void_p,
                                  c_void_p, c_int64, c_void_p, c_size_t, c_void_p]),
    "oomb_select_tiled_workspace_bytes": (c_size_t, [P_pool, c_int32, c_int64, c_int32]),
    "oomb_select_pages_tiled": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                        c_int32, c_int64, c_int32, c_int32, c_void_p, c_int64,
                                        c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_size_t,
                                        c_void_p]),
    "oomb_select_pages_noalloc": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                          c_int32, c_int64, c_int32, c_void_p, c_int64, c_void_p,
                                          c_void_p, c_void_p, c_int64, c_void_p]),
    "oomb_rope": (c_int, [c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64, c_int32, c_int32,
                          c_int32, c_int32, c_int64, c_float, c_int32, c_void_p]),
    "oomb_page_summarize_mean": (c_int, [P_pool, c_void_p, c_int64, c_int64, c_int64, c_int64,
                                         c_void_p, c_void_p]),
    "oomb_select_pages_mean": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                       c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int64,
                                       c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_size_t,
                                       c_void_p]),
    "oomb_paged_chunk_attn_fwd": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                          c_int32, c_int64, c_void_p, c_int64, c_void_p, c_int32,
                                          c_float,
                                          c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                          c_size_t, c_void_p]),
    "oomb_fwd_workspace_bytes": (c_size_t, [P_pool, c_int32, c_int64, c_int64, c_int32]),
    "oomb_bwd_workspace_bytes": (c_size_t, [P_pool, c_int32, c_int64, c_int64, c_int32]),
    "oomb_split_plan": (c_int, [P_pool, c_int32, c_int64, c_int64, c_int32, ctypes.POINTER(c_int32)]),
    "oomb_copy_pages": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                                c_int32, c_void_p, c_void_p]),
    "oomb_copy_pages_sdma": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p,
                                     c_void_p, c_int32, c_void_p]),
    "oomb_add_pages_f32": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p,
                                   c_void_p, c_int32, c_void_p, c_int32, c_void_p]),
    "oomb_fetch_selected": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                    c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p,
                                    c_int64, c_int64, c_void_p]),
    "oomb_profile_enable": (c_int, [c_int]),
    "oomb_profile_collect": (c_int, [ctypes.POINTER(c_char_p), ctypes.POINTER(c_float), c_int]),
    "oomb_paged_chunk_attn_bwd": (c_int, [P_pool, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                          c_int64, c_int64, c_int32, c_int64, c_void_p, c_int64,
                                          c_void_p, c_int32, c_float, c_void_p, c_int64, c_int64,
                                          c_void_p,
                                          c_int64, c_int64, c_void_p, c_void_p, c_int64, c_int64,
                                          c_void_p, c_size_t, c_void_p]),
}

_lib = None


class OombError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_chunk_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def call(name: str, *args) -> int:
    status = getattr(lib(), name)(*args)
    if status != OOMB_OK:
        raise OombError(name, status, lib().oomb_last_error().decode())
    return status
