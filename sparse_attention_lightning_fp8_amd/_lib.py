"""ctypes loader for liblk.so (the HIP library behind include/lk.h).

There is no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

# The in-tree build; LK_LIB_PATH names another build of the same library (the CPU
# sanitizer tests load a host-instrumented copy through it).
LIB_PATH = os.environ.get("LK_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblk.so")

LK_OK = 0
STATUS_NAMES = {0: "LK_OK", -1: "LK_E_NULL", -2: "LK_E_SHAPE", -3: "LK_E_UNSUPPORTED", -4: "LK_E_HIP",
                -5: "LK_E_SCRATCH"}

# Every function the header declares, as (name, restype, argtypes).
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class LkRows(ctypes.Structure):
    """Mirror of `lk_rows` in include/lk.h."""
    _fields_ = [("B", _i32), ("S", _i32), ("T", _i64), ("start_pos", _i64),
                ("seq_len", _p), ("causal", _i32)]


SIGNATURES = {
    "lk_quantize_keys": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _i64, _i64, _i64, _p, _p]),
    "lk_quantize_queries": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _p, _p, _p]),
    "lk_prepare": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _i64, _i64, _i64, _p,
                                  _p, _p, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _p]),
    "lk_index_score": (ctypes.c_int, [_p, _p, _i32, _p, _p, _i64, ctypes.POINTER(LkRows), _p, _p]),
    "lk_decode_score": (ctypes.c_int, [_p, _p, _i32, _p, _p, _p, _i64, ctypes.POINTER(LkRows), _p, _p, _p,
                                       _p, _p, _p]),
    "lk_decode_select": (ctypes.c_int, [_p, _p, _i32, _p, _p, _p, _i64, ctypes.POINTER(LkRows), _p, _p, _p,
                                        _p, _p, _i32, _p, _p]),
    "lk_topk": (ctypes.c_int, [_p, ctypes.POINTER(LkRows), _i32, _p, _p]),
    "lk_sparse_mla_workspace_size": (ctypes.c_size_t, [_i32, _i32]),
    "lk_sparse_mla_decode": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _p, _i32, _i32, ctypes.c_float, _p, _p,
                                            ctypes.c_size_t, _p]),
    "lk_sparse_mla_decode_static": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _p, _i32, _i32, ctypes.c_float,
                                                   _p, _p]),
    "lk_probe_empty": (ctypes.c_int, [_i32, _p]),
    "lk_probe_read": (ctypes.c_int, [_p, ctypes.c_size_t, _p, _i32, _p]),
    "lk_probe_fp8_mfma_score": (ctypes.c_int, [_p, _p, _p, _p, _i64, ctypes.POINTER(LkRows), _p, _p]),
    "lk_profile_next_launch": (ctypes.c_int, [_p, _p]),
    "lk_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lk_abi_version": (_i32, []),
}

_lib = None


class LkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with every declared signature set; raise if
    it is not built or its ABI version differs."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python sparse_attention_lightning_fp8_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.lk_abi_version() != 1:
        raise ImportError(f"{path}: unexpected ABI version {lib.lk_abi_version()}")
    return lib


def load() -> ctypes.CDLL:
    """Load liblk.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def status_string(status: int) -> str:
    try:
        return load().lk_status_string(status).decode()
    except ImportError:
        return STATUS_NAMES.get(status, "unknown")


def check(fn: str, status: int) -> None:
    if status != LK_OK:
        raise LkError(fn, status)
