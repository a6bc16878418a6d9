"""ctypes loader of libglance.so: the C ABI of include/glance.h, names unchanged.

Argument marshalling only.  The library must be built (``build.py``); a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libglance.so")

GLANCE_F32 = 0
GLANCE_BF16 = 1
GLANCE_MAX_L = 16
GLANCE_MAX_ROWS = 64
STATUS = {0: "GLANCE_OK", -1: "GLANCE_ERR_INVALID_ARG", -2: "GLANCE_ERR_ALIGNMENT",
          -3: "GLANCE_ERR_WORKSPACE", -4: "GLANCE_ERR_UNSUPPORTED", -5: "GLANCE_ERR_HIP"}

_P = ctypes.c_void_p
_I = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_U64 = ctypes.c_uint64


class GlanceAttnLayer(ctypes.Structure):
    _fields_ = [("wq", _P), ("wk", _P), ("wv", _P), ("wo", _P), ("k_cache", _P), ("v_cache", _P),
                ("packed", _P)]


class GlanceFullLayer(ctypes.Structure):
    _fields_ = [("attn", GlanceAttnLayer), ("g_attn", _P), ("g_q", _P), ("g_k", _P), ("g_mlp", _P),
                ("w_gate", _P), ("w_up", _P), ("w_down", _P), ("inter", _I), ("eps", _F),
                ("mlp_packed", _P)]


class GlanceWalk(ctypes.Structure):
    _fields_ = [("parent", _P), ("token", _P), ("n_valid", _P), ("nseq", _I), ("n_rows", _I),
                ("L", _I), ("gap_flag", _F), ("n_accept", _P), ("out_tokens", _P),
                ("path_rows", _P), ("flagged", _P)]


# name -> (restype, argtypes), exactly the declarations of include/glance.h
SIGNATURES = {
    "glance_build_tree": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "glance_build_tree_ws": (_SZ, [_I, _I, _I, _I]),
    "glance_build_tree_flag_offset": (_SZ, [_I, _I, _I, _I]),
    "glance_entropy_log_value": (_I, [_P, _I, _I, _F, _F, _I, _P, _P]),
    "glance_build_tree_shared": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P,
                                      _P, _P, _SZ, _P]),
    "glance_tree_attn": (_I, [ctypes.POINTER(GlanceAttnLayer), _I, _P, _P, _P, _P, _P, _I64,
                              _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ,
                              _P]),
    "glance_tree_attn_ws": (_SZ, [_I, _I, _I64, _I, _I, _I, _I]),
    "glance_tree_layer": (_I, [ctypes.POINTER(GlanceFullLayer), _P, _P, _P, _P, _P, _I64, _P, _P,
                               _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "glance_tree_layer_ws": (_SZ, [_I, _I, _I64, _I, _I, _I, _I, _I]),
    "glance_mlp_pack_bytes": (_SZ, [_I, _I]),
    "glance_mlp_pack": (_I, [_P, _P, _P, _I, _I, _P, _P]),
    "glance_verify_head": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "glance_verify_head_ws": (_SZ, [_I, _I, _I, _I]),
    "glance_verify_head_sampled": (_I, [_P, _P, _I, _I, _I, _I, _F, _U64, _U64, _P, _P, _P, _P,
                                        _P, _P, _P, _P, _SZ, _P]),
    "glance_head_pack_bytes": (_SZ, [_I, _I]),
    "glance_head_pack": (_I, [_P, _I, _I, _P, _P]),
    "glance_attn_pack_bytes": (_SZ, [_I, _I, _I, _I]),
    "glance_attn_pack": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "glance_verify_head_packed": (_I, [_P, _P, _I, _I, _I, _F, _U64, _U64, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _SZ, _P]),
    "glance_verify_head_walk": (_I, [_P, _P, _I, _I, _I, _F, _U64, _U64, _P, _P, _P, _P, _P, _P,
                                     _P, ctypes.POINTER(GlanceWalk), _P, _SZ, _P]),
    "glance_verify_head_packed_noalloc": (_I, [_P, _P, _I, _I, _I, _F, _U64, _U64, _P, _P, _P, _P,
                                               _P, _P, _P, _P]),
    "glance_accept_walk": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P]),
    "glance_commit_kv": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I64, _P]),
    "glance_advance_round": (_I, [_P, _P, _I, _P, _P, _P]),
    "glance_head_timing": (_I, [_P, _P]),
    "glance_read_probe": (_I, [_P, _SZ, _I, _P, _P]),
    "glance_status_string": (ctypes.c_char_p, [_I]),
    "glance_last_error": (ctypes.c_char_p, []),
    "glance_abi_version": (_I, []),
}

_lib = None


class GlanceError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libglance.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tree_verified_block_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        detail = load().glance_last_error().decode()
        raise GlanceError(fn, status, detail)


def call(fn: str, *args) -> None:
    """Call a status-returning entry point and raise GlanceError on failure."""
    check(fn, getattr(load(), fn)(*args))
