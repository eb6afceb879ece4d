"""The C ABI on the host: the library loads, exports every symbol include/lk.h declares,
and every validation error returns before any HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from sparse_attention_lightning_fp8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lk.h")

OK, E_NULL, E_SHAPE, E_UNSUP = 0, -1, -2, -3
A = 0x10000  # a 16-byte aligned fake device address: never dereferenced by these calls


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LK_API\s+[\w\s\*]+?\b(lk_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    assert syms == sorted(["lk_quantize_keys", "lk_quantize_queries", "lk_index_score", "lk_topk",
                           "lk_prepare", "lk_decode_score", "lk_decode_select", "lk_sparse_mla_workspace_size",
                           "lk_sparse_mla_decode", "lk_sparse_mla_decode_static", "lk_profile_next_launch",
                           "lk_probe_empty", "lk_probe_read", "lk_probe_fp8_mfma_score", "lk_status_string",
                           "lk_abi_version"])


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert set(declared_symbols()) == set(_lib.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    assert lib.lk_abi_version() == 1
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.lk_status_string(code).decode().startswith(name)
    assert lib.lk_status_string(7).decode() == "unknown lk_status"


def rows(B=1, S=1, T=16, start=0, seq_len=None, causal=0):
    return ctypes.byref(_lib.LkRows(B, S, T, start, seq_len, causal))


def test_quantize_keys_validation(lib):
    f = lib.lk_quantize_keys
    assert f(A, -1, 1, 1, A, A, 16, 16, 0, None, None) == E_SHAPE
    assert f(A, 1, 1, 1, A, A, 16, 17, 0, None, None) == E_SHAPE         # cache_rows > stride
    assert f(None, 1, 1, 1, A, A, 16, 16, 0, None, None) == E_NULL
    assert f(A, 1, 1, 1, None, A, 16, 16, 0, None, None) == E_NULL
    assert f(A, 1, 1, 1, A, None, 16, 16, 0, None, None) == E_NULL
    assert f(A + 8, 1, 1, 1, A, A, 16, 16, 0, None, None) == E_UNSUP     # misaligned bf16 rows
    assert f(A, 1, 1, 1, A + 4, A, 16, 16, 0, None, None) == E_UNSUP
    assert f(A, 1, 1, 1, A, A, 16, 16, 0, A + 2, None) == E_UNSUP        # misaligned positions
    assert f(None, 0, 5, 0, None, None, 0, 0, 0, None, None) == OK        # empty: nothing to do
    # a host-known destination must fit the cache: rows [row_offset, row_offset + n_rows)
    assert f(A, 2, 5, 5, A, A, 16, 16, 12, None, None) == E_SHAPE         # 12 + 5 > 16
    assert f(A, 1, 17, 17, A, A, 16, 16, 0, None, None) == E_SHAPE        # more rows than the cache
    assert f(A, 1, 1, 1, A, A, 16, 16, -1, None, None) == E_SHAPE         # negative offset
    assert f(A, 1, 1, 1, A, A, 16, 16, 1 << 62, None, None) == E_SHAPE    # no overflow in the check
    # device positions are the kernel's to check (rows outside the cache are skipped):
    # the same sizes pass validation and only then fail on the fake pointers' alignment
    assert f(A, 2, 5, 5, A, A, 16, 16, 12, A + 2, None) == E_UNSUP


def test_quantize_queries_validation(lib):
    f = lib.lk_quantize_queries
    assert f(A, A, -1, 64, A, A, None, None) == E_SHAPE
    assert f(A, A, 1, 0, A, A, None, None) == E_SHAPE
    assert f(None, A, 1, 64, A, A, None, None) == E_NULL
    assert f(A, None, 1, 64, A, A, None, None) == E_NULL
    assert f(A, A, 1, 64, None, A, None, None) == E_NULL
    assert f(A, A, 1, 64, A, None, None, None) == E_NULL
    assert f(A, A, 1, 64, A + 4, A, None, None) == E_UNSUP
    assert f(A, A, 1, 64, A, A, A + 1, None) == E_UNSUP
    assert f(None, None, 0, 64, None, None, None, None) == OK


def test_prepare_validation(lib):
    f = lib.lk_prepare
    K = (A, 1, 1, 1, A, A, 16, 16, 0, None)
    Q = (A, A, 1, 64, A, A, None)
    R = (None, None, None, None)
    assert f(A, -1, 1, 1, A, A, 16, 16, 0, None, *Q, *R, None) == E_SHAPE
    assert f(*K, A, A, -1, 64, A, A, None, *R, None) == E_SHAPE
    assert f(*K, None, A, 1, 64, A, A, None, *R, None) == E_NULL
    assert f(None, 1, 1, 1, A, A, 16, 16, 0, None, *Q, *R, None) == E_NULL
    assert f(*K, A + 4, A, 1, 64, A, A, None, *R, None) == E_UNSUP
    assert f(*K, *Q, A, None, None, None, None) == E_NULL                  # RoPE tables come in pairs
    assert f(*K, *Q, None, None, None, A, None) == E_NULL
    assert f(*K, *Q, A + 4, A, None, None, None) == E_UNSUP                # misaligned table
    assert f(None, 0, 0, 0, None, None, 0, 0, 0, None, None, None, 0, 64, None, None, None, *R, None) == OK


def test_index_score_validation(lib):
    f = lib.lk_index_score
    assert f(A, A, 64, A, A, 16, None, A, None) == E_NULL
    assert f(A, A, 64, A, A, 16, rows(B=-1), A, None) == E_SHAPE
    assert f(A, A, 64, A, A, 16, rows(T=17), A, None) == E_SHAPE             # T beyond the cache
    assert f(A, A, 32, A, A, 16, rows(), A, None) == E_UNSUP                 # heads != 64
    assert f(None, A, 64, A, A, 16, rows(), A, None) == E_NULL
    assert f(A, A, 64, None, A, 16, rows(), A, None) == E_NULL
    assert f(A, A, 64, A, A, 16, rows(), None, None) == E_NULL
    assert f(A + 8, A, 64, A, A, 16, rows(), A, None) == E_UNSUP
    assert f(A, A + 4, 64, A, A, 16, rows(), A, None) == E_UNSUP
    assert f(A, A, 64, A, A, 16, rows(seq_len=A + 1), A, None) == E_UNSUP
    assert f(A, A, 64, A, A, 70000, rows(B=70000, T=16), A, None) == E_UNSUP  # grid limit
    # prefill grid: one block per (sequence, 8-token group, 4096-key slice), at most 2^31 - 1
    assert f(A, A, 64, A, A, 16, rows(B=65535, S=1 << 27, T=16), A, None) == E_UNSUP
    assert f(A, A, 64, A, A, 16, rows(S=4 * 65535, T=16, seq_len=A + 2), A, None) == E_UNSUP   # misaligned
    assert f(None, None, 64, None, None, 16, rows(B=0), None, None) == OK
    assert f(None, None, 64, None, None, 16, rows(T=0), None, None) == OK


def test_decode_score_validation(lib):
    f = lib.lk_decode_score
    #       q  w   H   kn k_cache k_scale stride rows      scores q8o  weo  cos sin stream
    assert f(A, A, 64, A, A, A, 16, None, A, None, None, None, None, None) == E_NULL
    assert f(A, A, 64, A, A, A, 16, rows(S=2), A, None, None, None, None, None) == E_SHAPE      # decode rows only
    assert f(A, A, 64, A, A, A, 16, rows(T=17), A, None, None, None, None, None) == E_SHAPE     # T beyond the cache
    assert f(A, A, 32, A, A, A, 16, rows(), A, None, None, None, None, None) == E_UNSUP         # heads != 64
    assert f(A, A, 64, A, A, A, 16, rows(), A, A, None, None, None, None) == E_NULL             # one optional output
    assert f(None, A, 64, A, A, A, 16, rows(), A, None, None, None, None, None) == E_NULL
    assert f(A, A, 64, None, A, A, 16, rows(), A, None, None, None, None, None) == E_NULL
    assert f(A, A, 64, A, A, A, 16, rows(), None, None, None, None, None, None) == E_NULL
    assert f(A + 8, A, 64, A, A, A, 16, rows(), A, None, None, None, None, None) == E_UNSUP     # misaligned q
    assert f(A, A, 64, A + 8, A, A, 16, rows(), A, None, None, None, None, None) == E_UNSUP     # misaligned k_new
    assert f(A, A + 2, 64, A, A, A, 16, rows(), A, None, None, None, None, None) == E_UNSUP
    assert f(A, A, 64, A, A, A, 16, rows(), A, A + 4, A, None, None, None) == E_UNSUP
    assert f(A, A, 64, A, A, A, 70000, rows(B=70000, T=16), A, None, None, None, None, None) == E_UNSUP
    assert f(A, A, 64, A, A, A, 16, rows(), A, None, None, A, None, None) == E_NULL     # RoPE pair
    assert f(A, A, 64, A, A, A, 16, rows(), A, None, None, A + 8, A, None) == E_UNSUP
    assert f(None, None, 64, None, None, None, 16, rows(B=0), None, None, None, None, None, None) == OK


def test_decode_select_validation(lib):
    f = lib.lk_decode_select
    #   q  w   H   kn k_cache k_scale stride rows  scores q8o  weo  cos  sin  k  idx stream
    def c(q=A, w=A, H=64, kn=A, kc=A, ks=A, stride=16, r=None, sc=A, q8o=None, weo=None, cos=None, sin=None,
          k=8, idx=A):
        return f(q, w, H, kn, kc, ks, stride, rows() if r is None else r, sc, q8o, weo, cos, sin, k, idx, None)
    assert f(A, A, 64, A, A, A, 16, None, A, None, None, None, None, 8, A, None) == E_NULL
    assert c(r=rows(S=2)) == E_SHAPE                                         # decode rows only
    assert c(r=rows(T=17)) == E_SHAPE                                        # T beyond the cache
    assert c(k=0) == E_SHAPE
    assert c(k=17) == E_SHAPE                                                # k beyond the row
    assert c(H=32) == E_UNSUP
    assert c(r=rows(T=16385), stride=16385) == E_UNSUP                       # beyond one top-k row
    assert c(q8o=A) == E_NULL                                                # one optional output
    assert c(q=None) == E_NULL
    assert c(idx=None) == E_NULL
    assert c(cos=A) == E_NULL                                                # RoPE tables come in pairs
    # scores may be left out only where the whole step is one launch (T <= 1024)
    assert c(sc=None, r=rows(T=1025), stride=1025, idx=A + 2) == E_NULL
    assert c(sc=None, idx=A + 2) == E_UNSUP                                  # passes the NULL check, misaligned idx
    assert c(q=A + 8) == E_UNSUP
    assert c(sc=A + 2) == E_UNSUP
    assert c(r=rows(B=70000, T=16)) == E_UNSUP                               # grid limit
    assert c(q=None, w=None, kn=None, kc=None, ks=None, sc=None, idx=None, r=rows(B=0)) == OK


def test_topk_validation(lib):
    f = lib.lk_topk
    assert f(A, None, 8, A, None) == E_NULL
    assert f(A, rows(), 0, A, None) == E_SHAPE
    assert f(A, rows(T=16), 17, A, None) == E_SHAPE                          # k beyond the row (k <= T)
    assert f(A, rows(S=-2), 8, A, None) == E_SHAPE
    assert f(A, rows(T=16385), 8, A, None) == E_UNSUP
    assert f(None, rows(), 8, A, None) == E_NULL
    assert f(A, rows(), 8, None, None) == E_NULL
    assert f(A + 2, rows(), 8, A, None) == E_UNSUP
    assert f(None, rows(B=0), 8, None, None) == OK


def test_sparse_mla_validation(lib):
    f = lib.lk_sparse_mla_decode
    ws = lib.lk_sparse_mla_workspace_size(16, 2048)
    assert ws == 16 * 8 * 128 * 514 * 4
    assert lib.lk_sparse_mla_workspace_size(0, 5) == 0
    #        qlat qrope kvl kvr stride cap  idx  B   n    scale out ws  wsb  stream
    assert f(A, A, A, A, 16, 17, A, 1, 8, 0.1, A, A, ws, None) == E_SHAPE       # cap beyond the stride
    assert f(A, A, A, A, 16, 16, A, -1, 8, 0.1, A, A, ws, None) == E_SHAPE
    assert f(A, A, A, A, 16, 16, A, 1, 8, 0.1, A, A, 10, None) == E_SHAPE       # workspace too small
    assert f(None, A, A, A, 16, 16, A, 1, 8, 0.1, A, A, ws, None) == E_NULL
    assert f(A, A, None, A, 16, 16, A, 1, 8, 0.1, A, A, ws, None) == E_NULL
    assert f(A, A, A, A, 16, 16, A, 1, 8, 0.1, A, None, ws, None) == E_NULL
    assert f(A + 8, A, A, A, 16, 16, A, 1, 8, 0.1, A, A, ws, None) == E_UNSUP
    assert f(A, A, A, A, 16, 16, A + 2, 1, 8, 0.1, A, A, ws, None) == E_UNSUP
    assert f(A, A, A, A, 16, 16, A, 70000, 8, 0.1, A, A, 1 << 40, None) == E_UNSUP   # grid limit
    assert f(A, A, A, A, 16, 16, A, 60000, 25600, 0.1, A, A, 1 << 45, None) == E_UNSUP   # 6e6 blocks
    assert f(A, A, A, A, 16, 16, A, 60000, 256, 0.1, A, A, 0, None) == E_SHAPE   # fits the grid, checks go on
    assert f(None, None, None, None, 16, 16, None, 0, 8, 0.1, None, None, 0, None) == OK


def test_sparse_mla_static_validation(lib):
    f = lib.lk_sparse_mla_decode_static
    #        qlat qrope kvl kvr stride cap  idx  B   n    scale out stream
    assert f(A, A, A, A, 16, 17, A, 1, 8, 0.1, A, None) == E_SHAPE              # cap beyond the stride
    assert f(A, A, A, A, 16, 16, A, 1, -8, 0.1, A, None) == E_SHAPE
    assert f(None, A, A, A, 16, 16, A, 1, 8, 0.1, A, None) == E_NULL
    assert f(A, A, A, A, 16, 16, None, 1, 8, 0.1, A, None) == E_NULL
    assert f(A, A, A, A + 8, 16, 16, A, 1, 8, 0.1, A, None) == E_UNSUP
    assert f(A, A, A, A, 16, 16, A, 70000, 8, 0.1, A, None) == E_UNSUP          # grid limit
    # beyond the 64 MiB static buffer (B = 32 rows of 2048 entries need 67.4 MB): refused
    assert lib.lk_sparse_mla_workspace_size(32, 2048) > (64 << 20)
    assert lib.lk_sparse_mla_workspace_size(16, 2048) <= (64 << 20)
    assert f(A, A, A, A, 16384, 16384, A, 32, 2048, 0.1, A, None) == -5         # LK_E_SCRATCH
    assert lib.lk_status_string(-5).decode().startswith("LK_E_SCRATCH")
    assert f(None, None, None, None, 16, 16, None, 0, 8, 0.1, None, None) == OK


def test_probe_validation(lib):
    assert lib.lk_probe_empty(0, None) == E_SHAPE
    assert lib.lk_probe_read(A, 24, A, 4, None) == E_SHAPE                   # not a multiple of 16
    assert lib.lk_probe_read(A, 32, A, 0, None) == E_SHAPE
    assert lib.lk_probe_read(None, 32, A, 4, None) == E_NULL
    assert lib.lk_probe_read(A + 8, 32, A, 4, None) == E_UNSUP
    assert lib.lk_probe_read(None, 0, None, 4, None) == OK
    f = lib.lk_probe_fp8_mfma_score
    assert f(A, A, A, A, 16, rows(S=2), A, None) == E_SHAPE                  # decode rows only
    assert f(A, A, A, A, 16, rows(T=17), A, None) == E_SHAPE
    assert f(None, A, A, A, 16, rows(), A, None) == E_NULL
    assert f(A + 4, A, A, A, 16, rows(), A, None) == E_UNSUP
    assert f(None, None, None, None, 16, rows(B=0), None, None) == OK


def test_profile_next_launch_validation(lib):
    assert lib.lk_profile_next_launch(None, A) == E_NULL
    assert lib.lk_profile_next_launch(A, None) == E_NULL
    # arming fake handles and then failing validation consumes them without any HIP call
    assert lib.lk_profile_next_launch(A, A) == OK
    assert lib.lk_topk(A, rows(), 0, A, None) == E_SHAPE


def test_python_binding_raises_without_gpu_tensors():
    import torch
    from sparse_attention_lightning_fp8_amd import api
    with pytest.raises(ValueError):
        api.lk_topk(torch.zeros(1, 1, 4, dtype=torch.float64), 2)
    with pytest.raises(ValueError):
        api.lk_quantize_queries(torch.zeros(2, 64, 128, dtype=torch.float32), torch.zeros(2, 64))
