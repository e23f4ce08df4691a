"""ctypes loader for ``libpkv.so`` (argument marshalling only).

The library is built in-tree by ``paged_attention_slot_amd.build``.  There is
no fallback: if the shared object is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

c_i32, c_i64, c_size, c_float, c_void_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                            ctypes.c_float, ctypes.c_void_p)
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_NO_FREE_BLOCKS, PKV_ERR_HIP = range(5)
PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = 0, 1, 2, 3
PKV_ROUTE_PARTITIONS, PKV_ROUTE_BALANCED, PKV_ROUTE_MATRIX, PKV_ROUTE_MATRIX_BALANCED = 0, 1, 2, 3
PKV_NOALLOC_SCRATCH_BYTES = 64 << 20


class PkvGeom(ctypes.Structure):
    _fields_ = [("num_blocks", c_i32), ("block_size", c_i32), ("num_kv_heads", c_i32),
                ("head_dim", c_i32), ("dtype", c_i32)]


class PkvKvScales(ctypes.Structure):
    _fields_ = [("k_scale", c_float), ("v_scale", c_float), ("k_scales", c_void_p),
                ("v_scales", c_void_p)]


# name -> (restype, argtypes); mirrors include/pkv.h
class PkvHostPool(ctypes.Structure):
    _fields_ = [("num_blocks", c_i32), ("k", c_void_p), ("v", c_void_p), ("k_scales", c_void_p),
                ("v_scales", c_void_p)]


SIGNATURES = {
    "pkv_version": (c_i32, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_set_tuning": (c_i32, [ctypes.c_char_p, c_i32]),
    "pkv_get_tuning": (c_i32, [ctypes.c_char_p]),
    "pkv_write": (c_i32, [c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_void_p,
                          ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_copy_blocks": (c_i32, [c_void_p, c_i32, c_void_p, c_void_p, ctypes.POINTER(PkvGeom),
                                c_void_p]),
    "pkv_write_quant": (c_i32, [c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_void_p,
                                ctypes.POINTER(PkvKvScales), ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_copy_blocks_quant": (c_i32, [c_void_p, c_i32, c_void_p, c_void_p,
                                      ctypes.POINTER(PkvKvScales), ctypes.POINTER(PkvGeom),
                                      c_void_p]),
    "pkv_attention_decode_quant": (c_i32, [c_i32, c_void_p, c_void_p, c_void_p,
                                           ctypes.POINTER(PkvKvScales), c_void_p, c_i32,
                                           c_void_p, c_float, c_void_p, c_i32, c_i32, c_i32,
                                           c_i32, c_void_p, c_size, ctypes.POINTER(PkvGeom),
                                           c_void_p]),
    "pkv_attention_multi_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                     ctypes.POINTER(PkvGeom)]),
    "pkv_attention_multi": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                    c_void_p, c_float, c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                    c_i32, c_void_p, c_size, ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_attention_partition_tokens": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(PkvGeom)]),
    "pkv_attention_piece_tokens": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(PkvGeom)]),
    "pkv_attention_decode_route": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(PkvGeom)]),
    "pkv_attention_decode_append_folded": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32,
                                                    ctypes.POINTER(PkvGeom)]),
    "pkv_attention_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32,
                                               ctypes.POINTER(PkvGeom)]),
    "pkv_attention_decode": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_void_p,
                                     c_float, c_void_p, c_i32, c_i32, c_i32, c_i32, c_void_p,
                                     c_size, ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_attention_decode_noalloc": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                             c_void_p, c_float, c_void_p, c_i32, c_i32, c_i32,
                                             c_i32, ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_attention_decode_phase": (c_i32, [c_i32, c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                           c_void_p, c_float, c_void_p, c_i32, c_i32, c_i32,
                                           c_i32, c_void_p, c_size, ctypes.POINTER(PkvGeom),
                                           c_void_p]),
    "pkv_attention_decode_append": (c_i32, [c_i32, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_i32, c_void_p,
                                            c_float, c_void_p, c_i32, c_i32, c_i32, c_i32,
                                            c_void_p, c_size, ctypes.POINTER(PkvGeom),
                                            c_void_p]),
    "pkv_stream_read": (c_i32, [c_void_p, c_size, c_void_p, c_i32, c_void_p]),
    "pkv_bm_create": (c_void_p, [c_i32, c_i32, P_i32]),
    "pkv_bm_destroy": (None, [c_void_p]),
    "pkv_bm_add_seq": (c_i32, [c_void_p, c_i64]),
    "pkv_bm_share_prefix": (c_i32, [c_void_p, c_i64, c_i64, c_i32]),
    "pkv_bm_fork": (c_i32, [c_void_p, c_i64, c_i64]),
    "pkv_bm_append_slots": (c_i32, [c_void_p, P_i64, c_i32, c_i32, P_i32, P_i32, P_i32]),
    "pkv_bm_free_seq": (c_i32, [c_void_p, c_i64]),
    "pkv_bm_export": (c_i32, [c_void_p, P_i64, c_i32, c_i32, P_i32, P_i32]),
    "pkv_bm_num_free": (c_i32, [c_void_p]),
    "pkv_bm_refcount": (c_i32, [c_void_p, c_i32]),
    "pkv_bm_num_tokens": (c_i32, [c_void_p, c_i64]),
    "pkv_bm_free_list": (c_i32, [c_void_p, P_i32, c_i32, P_i32]),
    "pkv_bm_check": (c_i32, [c_void_p]),
    "pkv_swap_out": (c_i32, [c_void_p, c_i32, c_void_p, c_void_p, ctypes.POINTER(PkvKvScales),
                             ctypes.POINTER(PkvHostPool), ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_swap_in": (c_i32, [c_void_p, c_i32, ctypes.POINTER(PkvHostPool), c_void_p, c_void_p,
                            ctypes.POINTER(PkvKvScales), ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_attention_shared_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                      c_i32, ctypes.POINTER(PkvGeom)]),
    "pkv_attention_decode_shared": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                            c_void_p, c_void_p, c_void_p, c_i32, c_i32, c_i32,
                                            c_i32, c_float, c_void_p, c_i32, c_i32, c_i32,
                                            c_void_p, c_size, ctypes.POINTER(PkvGeom), c_void_p]),
    "pkv_prefix_groups": (c_i32, [P_i32, c_i32, c_i32, P_i32, c_i32, P_i32, P_i32, P_i32, P_i32,
                                  P_i32, P_i32]),
    "pkv_attention_multi_quant": (c_i32, [c_void_p, c_void_p, c_void_p, c_void_p,
                                          ctypes.POINTER(PkvKvScales), c_void_p, c_i32, c_void_p,
                                          c_float, c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          c_i32, c_void_p, c_size, ctypes.POINTER(PkvGeom),
                                          c_void_p]),
    "pkv_attention_decode_shared_quant": (c_i32, [c_void_p, c_void_p, c_void_p,
                                                  ctypes.POINTER(PkvKvScales), c_void_p, c_i32,
                                                  c_void_p, c_void_p, c_void_p, c_i32, c_i32, c_i32,
                                                  c_i32, c_float, c_void_p, c_i32, c_i32, c_i32,
                                                  c_void_p, c_size, ctypes.POINTER(PkvGeom),
                                                  c_void_p]),
    "pkv_bm_add_host_pool": (c_i32, [c_void_p, c_i32, P_i32]),
    "pkv_bm_swap_out": (c_i32, [c_void_p, P_i64, c_i32, P_i32, c_i32, P_i32]),
    "pkv_bm_swap_in": (c_i32, [c_void_p, P_i64, c_i32, P_i32, c_i32, P_i32]),
    "pkv_bm_distinct_blocks": (c_i32, [c_void_p, P_i64, c_i32]),
    "pkv_bm_is_swapped": (c_i32, [c_void_p, c_i64]),
    "pkv_bm_num_free_host": (c_i32, [c_void_p]),
    "pkv_bm_host_refcount": (c_i32, [c_void_p, c_i32]),
    "pkv_bm_host_free_list": (c_i32, [c_void_p, P_i32, c_i32, P_i32]),
}

_lock = threading.Lock()
_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run "
                                  "`python -m paged_attention_slot_amd.build` first")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where, lib().pkv_last_error().decode(errors="replace"))
