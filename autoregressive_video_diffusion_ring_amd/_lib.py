"""ctypes view of librc.so (include/rc.h): the struct, the enums, the symbols.

Argument marshalling only.  There is no fallback: if the library is not built
the import of any entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librc.so")

RC_OK, RC_ERR_ARG, RC_ERR_UNSUPPORTED, RC_ERR_STATE, RC_ERR_HIP = range(5)
RC_F32, RC_BF16, RC_FP8_E4M3 = range(3)
RC_MASK_BLOCK_CAUSAL, RC_MASK_SAME_BLOCK = range(2)
RC_PRECISION_AUTO, RC_PRECISION_TWO_TERM, RC_PRECISION_ONE_TERM = range(3)
STATUS_NAMES = {0: "RC_OK", 1: "RC_ERR_ARG", 2: "RC_ERR_UNSUPPORTED", 3: "RC_ERR_STATE", 4: "RC_ERR_HIP"}
DTYPES = {"f32": RC_F32, "bf16": RC_BF16, "fp8": RC_FP8_E4M3}


class RcRing(ctypes.Structure):
    """Mirror of ``struct rc_ring``."""

    _fields_ = [
        ("n_slots", c_int32), ("n_heads", c_int32), ("head_dim", c_int32), ("kv_dtype", c_int32),
        ("rope_base", c_float), ("v_ld", c_int32), ("n_anchor", c_int32), ("n_memory", c_int32),
        ("k", c_void_p), ("v", c_void_p), ("k_scale", c_void_p), ("v_scale", c_void_p),
        ("slot_pos", c_void_p), ("slot_block", c_void_p),
        ("head", c_int32), ("n_hist", c_int32), ("n_cur", c_int32), ("cur_pos0", c_int32),
        ("cur_block", c_int32), ("n_mem", c_int32), ("max_block", c_int32),
        ("pos_lo", c_int32), ("pos_hi", c_int32),
    ]


class RcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None

# name -> (restype, argtypes), in the order of include/rc.h
SIGNATURES = {
    "rc_ring_v_ld": (c_int32, [c_int32]),
    "rc_ring_sizes": (c_int32, [c_int32, c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "rc_ring_init": (c_int32, [POINTER(RcRing), c_int32, c_void_p]),
    "rc_cache_write": (c_int32, [POINTER(RcRing), c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    "rc_cache_rerotate": (c_int32, [POINTER(RcRing), c_int32, c_void_p]),
    "rc_chunk_attention": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                     c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "rc_chunk_attention_ex": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                        c_int32, c_float, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "rc_set_attention_precision": (c_int32, [c_int32]),
    "rc_attention_workspace_bytes": (c_size_t, [POINTER(RcRing), c_int32]),
    "rc_chunk_attention_noalloc": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                             c_float, c_void_p, c_void_p, c_void_p]),
    "rc_attention_noalloc_limit": (c_size_t, []),
    "rc_qkv_project_write": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                       c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "rc_qkv_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "rc_ring_advance": (c_int32, [POINTER(RcRing), c_int32]),
    "rc_key_mass": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_int32, c_int32, c_float, c_float,
                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "rc_key_mass_slots": (c_int32, [POINTER(RcRing), c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                    c_float, c_void_p, POINTER(c_int32), c_int32, c_void_p, c_void_p, c_size_t,
                                    c_void_p]),
    "rc_key_mass_workspace_bytes": (c_size_t, [POINTER(RcRing), c_int32]),
    "rc_cache_write_scored": (c_int32, [POINTER(RcRing), c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                        c_float, c_void_p, c_size_t, c_void_p]),
    "rc_cache_write_scored_workspace_bytes": (c_size_t, [POINTER(RcRing), c_int32]),
    "rc_debug_visibility": (c_int32, [POINTER(RcRing), c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "rc_debug_tile_classes_bytes": (c_size_t, [POINTER(RcRing), c_int32]),
    "rc_debug_tile_classes": (c_int32, [POINTER(RcRing), c_int32, c_int32, c_int32, c_int32, c_float, c_void_p,
                                        c_size_t, c_void_p]),
    "rc_last_error": (c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """Load librc.so once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m autoregressive_video_diffusion_ring_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != RC_OK:
        raise RcError(status, lib().rc_last_error().decode())
