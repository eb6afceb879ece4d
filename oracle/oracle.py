"""Python access to the plain C oracle (lk_oracle.c).

TEST INFRASTRUCTURE ONLY: the product package never imports this module.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

Every function here is argument marshalling around one C routine, whose comment
cites the page passage it follows.  Arrays are numpy; bf16 data travels as its
uint16 bit pattern.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lk_oracle.c")
_LIB = os.path.join(_HERE, "liblk_oracle.so")

LKO_OK = 0


def build() -> str:
    """Compile lk_oracle.c with gcc (strict IEEE: no contraction, -O2)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


def build_sanitized(out_path: str) -> str:
    """The same library built with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts), for the CPU sanitizer tests.  Loading it needs gcc's libasan
    preloaded; ``LK_ORACLE_LIB=<out_path>`` makes ``lib()`` load it."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           _SRC, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("LK_ORACLE_LIB", _LIB)
        if path == _LIB and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.lko_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.lko_e4m3_decode.restype = ctypes.c_double
        L.lko_e4m3_encode.argtypes = [ctypes.c_double, p]
        L.lko_bf16_decode.argtypes = [ctypes.c_uint16]
        L.lko_bf16_decode.restype = ctypes.c_double
        L.lko_bf16_round.argtypes = [ctypes.c_double, p]
        L.lko_hadamard_entry.argtypes = [ctypes.c_int, ctypes.c_int]
        L.lko_rotation_scale.argtypes = [ctypes.c_int]
        L.lko_rotation_scale.restype = ctypes.c_double
        L.lko_rotate_row.argtypes = [p, ctypes.c_int, p]
        L.lko_scale_exponent.argtypes = [ctypes.c_double]
        L.lko_quantize_row.argtypes = [p, ctypes.c_int, p, p]
        L.lko_quantize_rows.argtypes = [p, i64, ctypes.c_int, p, p]
        L.lko_fold_weights.argtypes = [p, p, i64, ctypes.c_int, p]
        L.lko_rope_row.argtypes = [p, ctypes.c_int, ctypes.c_int, p, p, p]
        L.lko_sparse_mla_row.argtypes = [p, p, ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p, i64, p,
                                         ctypes.c_int, ctypes.c_double, p]
        L.lko_rope_quantize_rows.argtypes = [p, i64, ctypes.c_int, ctypes.c_int, p, p, i64, p, p]
        L.lko_fold_weights.restype = None
        L.lko_valid_len.argtypes = [i64, i64, ctypes.c_int, i64, i64]
        L.lko_valid_len.restype = i64
        L.lko_score_row.argtypes = [p, p, ctypes.c_int, ctypes.c_int, p, p, i64, i64, p]
        L.lko_score_row.restype = None
        L.lko_topk_f64.argtypes = [p, i64, ctypes.c_int, p]
        L.lko_topk_f32.argtypes = [p, i64, ctypes.c_int, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


class OracleRangeError(ValueError):
    """The input lies outside the oracle's exact contract."""


def _check(rc: int, what: str) -> None:
    if rc != LKO_OK:
        raise OracleRangeError(f"{what}: oracle status {rc}")


# ---- codecs ----------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().lko_e4m3_decode(int(c)) for c in codes.ravel()],
                    dtype=np.float64).reshape(codes.shape)


def e4m3_encode(v: float) -> int:
    out = ctypes.c_uint8()
    _check(lib().lko_e4m3_encode(float(v), ctypes.addressof(out)), "e4m3_encode")
    return out.value


def bf16_decode(bits: int) -> float:
    return lib().lko_bf16_decode(int(bits))


def bf16_round(p: float) -> int:
    out = ctypes.c_uint16()
    _check(lib().lko_bf16_round(float(p), ctypes.addressof(out)), "bf16_round")
    return out.value


def hadamard_entry(j: int, i: int) -> int:
    return lib().lko_hadamard_entry(j, i)


def rotation_scale(d: int) -> float:
    return lib().lko_rotation_scale(d)


def scale_exponent(amax: float) -> int:
    return lib().lko_scale_exponent(float(amax))


# ---- quantization ------------------------------------------------------------
def rotate_row(x_bf16_bits: np.ndarray) -> np.ndarray:
    """Pre-rounding rotation p = fl64(exact(H x) * d**-0.5) of one row."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    d = x.shape[-1]
    p = np.empty(d, dtype=np.float64)
    _check(lib().lko_rotate_row(_ptr(x), d, _ptr(p)), "rotate_row")
    return p


def quantize_rows(x_bf16_bits: np.ndarray):
    """act_quant(rotate_activation(x)) per row of the last dimension.

    Returns (codes uint8 [..., d], scales float32 [...])."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    d = x.shape[-1]
    n = x.size // d
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _check(lib().lko_quantize_rows(_ptr(x), n, d, _ptr(codes), _ptr(scales)), "quantize_rows")
    return codes, scales


def rope_row(x_bf16_bits: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray, rope_dim: int = 64) -> np.ndarray:
    """RoPE on the leading rope_dim features of one bf16 row (reading R12); bf16 bits out."""
    x = np.ascontiguousarray(x_bf16_bits, np.uint16)
    c = np.ascontiguousarray(cos_t, np.float32)
    s = np.ascontiguousarray(sin_t, np.float32)
    assert c.size >= rope_dim // 2 and s.size >= rope_dim // 2
    y = np.empty_like(x)
    _check(lib().lko_rope_row(_ptr(x), x.size, rope_dim, _ptr(c), _ptr(s), _ptr(y)), "rope_row")
    return y


def rope_quantize_rows(x_bf16_bits: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray,
                       rows_per_table_row: int = 1, rope_dim: int = 64):
    """RoPE then act_quant of [n, 128] bf16 rows; row r uses table row r // rows_per_table_row."""
    x = np.ascontiguousarray(x_bf16_bits, np.uint16).reshape(-1, 128)
    n = x.shape[0]
    c = np.ascontiguousarray(cos_t, np.float32).reshape(-1, rope_dim // 2)
    s = np.ascontiguousarray(sin_t, np.float32).reshape(-1, rope_dim // 2)
    assert c.shape[0] * rows_per_table_row >= n and s.shape == c.shape
    codes = np.empty((n, 128), np.uint8)
    scales = np.empty(n, np.float32)
    _check(lib().lko_rope_quantize_rows(_ptr(x), n, 128, rope_dim, _ptr(c), _ptr(s), rows_per_table_row,
                                        _ptr(codes), _ptr(scales)), "rope_quantize_rows")
    return codes, scales


def fold_weights(w: np.ndarray, q_scale: np.ndarray, d: int = 128) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    assert w.shape == q_scale.shape
    out = np.empty(w.shape, dtype=np.float32)
    lib().lko_fold_weights(_ptr(w), _ptr(q_scale), w.size, d, _ptr(out))
    return out


# ---- score and top-k -----------------------------------------------------------
def valid_len(T: int, seq_len_b: int, causal: bool, start_pos: int, t: int) -> int:
    return lib().lko_valid_len(T, seq_len_b, 1 if causal else 0, start_pos, t)


def score_row(q8_row: np.ndarray, w_eff_row: np.ndarray, k8_seq: np.ndarray,
              k_scale_seq: np.ndarray, T: int, L: int) -> np.ndarray:
    """Scores of one query token against keys [0, T) of its sequence (fp64).

    q8_row [H, d] uint8; w_eff_row [H] float32; k8_seq [>=T, d] uint8;
    k_scale_seq [>=T] float32."""
    q = np.ascontiguousarray(q8_row, dtype=np.uint8)
    w = np.ascontiguousarray(w_eff_row, dtype=np.float32)
    k = np.ascontiguousarray(k8_seq, dtype=np.uint8)
    ks = np.ascontiguousarray(k_scale_seq, dtype=np.float32)
    H, d = q.shape
    assert w.shape == (H,) and k.shape[1] == d and k.shape[0] >= T and ks.shape[0] >= T
    out = np.empty(T, dtype=np.float64)
    lib().lko_score_row(_ptr(q), _ptr(w), H, d, _ptr(k), _ptr(ks), T, L, _ptr(out))
    return out


def topk(values: np.ndarray, L: int, k: int) -> np.ndarray:
    """Indices of the min(k, L) largest values in values[:L] (ties: lower index),
    padded with -1; float32 and float64 inputs keep their own precision."""
    v = np.ascontiguousarray(values)
    out = np.empty(k, dtype=np.int32)
    if v.dtype == np.float32:
        rc = lib().lko_topk_f32(_ptr(v), L, k, _ptr(out))
    else:
        v = np.ascontiguousarray(v, dtype=np.float64)
        rc = lib().lko_topk_f64(_ptr(v), L, k, _ptr(out))
    _check(rc, "topk")
    return out


def sparse_mla_row(qc_bits: np.ndarray, qr_bits: np.ndarray, kv_bits: np.ndarray, pe_bits: np.ndarray,
                   idx: np.ndarray, scale: float) -> np.ndarray:
    """Sparse MLA decode attention of one row (reading R13): qc [H, Dc], qr [H, Dr] bf16
    bits, kv [T, Dc], pe [T, Dr] bf16 bits, idx int32 (-1 unused) -> float64 [H, Dc]."""
    qc = np.ascontiguousarray(qc_bits, np.uint16)
    qr = np.ascontiguousarray(qr_bits, np.uint16)
    kv = np.ascontiguousarray(kv_bits, np.uint16)
    pe = np.ascontiguousarray(pe_bits, np.uint16)
    ix = np.ascontiguousarray(idx, np.int32)
    H, Dc = qc.shape
    Dr = qr.shape[1]
    T = kv.shape[0]
    assert pe.shape == (T, Dr) and kv.shape[1] == Dc
    out = np.empty((H, Dc), np.float64)
    _check(lib().lko_sparse_mla_row(_ptr(qc), _ptr(qr), H, Dc, Dr, _ptr(kv), _ptr(pe), T, _ptr(ix), ix.size,
                                    float(scale), _ptr(out)), "sparse_mla_row")
    return out
