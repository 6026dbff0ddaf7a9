"""ctypes declarations of the C ABI in include/gva.h.

Loading fails loudly when libgva.so has not been built: there is no other
implementation of these operations in this package.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# GVA_LIBRARY names another build of the same library (for instance the
# host-sanitized one that the CPU test suite builds); default: the in-tree one.
LIB_PATH = os.environ.get("GVA_LIBRARY") or os.path.join(_PKG, "libgva.so")

GVA_OK = 0
GVA_ERR_INVALID_ARGUMENT = 1
GVA_ERR_UNSUPPORTED = 2
GVA_ERR_WORKSPACE = 3
GVA_ERR_HIP = 4

GVA_F32 = 0
GVA_BF16 = 1


class GvaShape(ctypes.Structure):
    """Mirror of `gva_shape` (all int32)."""

    _fields_ = [(name, ctypes.c_int32) for name in (
        "B", "H", "G", "d_n", "d_v", "d_r", "capacity", "max_seq_len", "block_size",
        "num_blocks", "max_blocks_per_seq", "split_tokens", "dtype")]

    def __repr__(self):
        return "GvaShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_shp = ctypes.POINTER(GvaShape)

# name -> (restype, argtypes); exactly the functions declared in include/gva.h
SIGNATURES = {
    "gva_append": (ctypes.c_int, [_shp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, ctypes.c_float, _vp]),
    "gva_rope_query": (ctypes.c_int, [_shp, _vp, _vp, _vp, ctypes.c_float, _vp]),
    "gva_decode": (ctypes.c_int, [_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                  _vp, ctypes.c_size_t, _vp]),
    "gva_decode_step": (ctypes.c_int, [_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_float, ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "gva_decode_step_workspace_bytes": (ctypes.c_size_t, [_shp]),
    "gva_decode_step_noalloc": (ctypes.c_int, [_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               ctypes.c_float, ctypes.c_float, _vp, _vp]),
    "gva_rope_query_multi": (ctypes.c_int, [_shp, _i32, _vp, _vp, _vp, ctypes.c_float, _vp]),
    "gva_decode_multi": (ctypes.c_int, [_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                        _vp, ctypes.c_size_t, _vp]),
    "gva_decode_multi_workspace_bytes": (ctypes.c_size_t, [_shp, _i32]),
    "gva_prefill": (ctypes.c_int, [_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "gva_copy_blocks": (ctypes.c_int, [_shp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gva_fork": (ctypes.c_int, [_shp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "gva_rollback": (ctypes.c_int, [_shp, _vp, _vp, _vp]),
    "gva_fold_query_projection": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "gva_query_projection": (ctypes.c_int, [_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gva_gqa_ref_decode": (ctypes.c_int, [_shp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                          ctypes.c_size_t, _vp]),
    "gva_decode_workspace_bytes": (ctypes.c_size_t, [_shp]),
    "gva_decode_split_tokens": (ctypes.c_int32, [_shp]),
    "gva_cache_bytes_per_token": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "gva_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gva_last_error": (ctypes.c_char_p, []),
    "gva_abi_version": (ctypes.c_int32, []),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"GVA HIP library not found at {path}; build it first with "
            "`python -m compact_kv_cache_amd._build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
