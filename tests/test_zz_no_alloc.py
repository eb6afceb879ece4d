"""lk_sparse_mla_decode_static (no caller workspace, no allocation) through the C ABI:
its output equals lk_sparse_mla_decode's with a caller workspace, bit for bit, on two
calls in a row (the second smaller, so stale partials from the first would show).
The size limit is checked on the host (test_abi)."""
import ctypes

import pytest
import torch

from sparse_attention_lightning_fp8_amd import _lib
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp):
    return [t.to(DEV).contiguous() for t in (inp.q_lat, inp.q_rope, inp.kv_lat, inp.kv_rope, inp.idx)]


def _call_both(inp, scale):
    lib = _lib.load()
    ql, qr, kl, kr, idx = _dev(inp)
    B, n = idx.shape
    cap = kl.shape[1]
    stride = kl.stride(0) // 512
    stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = lib.lk_sparse_mla_workspace_size(B, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    out_ws = torch.full((B, 128, 512), float("nan"), dtype=torch.float32, device=DEV)
    out_st = torch.full((B, 128, 512), float("nan"), dtype=torch.float32, device=DEV)
    st = lib.lk_sparse_mla_decode(ql.data_ptr(), qr.data_ptr(), kl.data_ptr(), kr.data_ptr(), stride, cap,
                                  idx.data_ptr(), B, n, ctypes.c_float(scale), out_ws.data_ptr(), ws.data_ptr(),
                                  ws.numel(), stream)
    _lib.check("lk_sparse_mla_decode", st)
    st = lib.lk_sparse_mla_decode_static(ql.data_ptr(), qr.data_ptr(), kl.data_ptr(), kr.data_ptr(), stride, cap,
                                         idx.data_ptr(), B, n, ctypes.c_float(scale), out_st.data_ptr(), stream)
    _lib.check("lk_sparse_mla_decode_static", st)
    torch.cuda.synchronize()
    return out_ws, out_st


def test_static_workspace_matches_caller_workspace():
    big = W.make_mla_inputs(W.MLA_WORKLOADS["mla_decode_b16_t16384"], seed=21)
    log("[no-alloc] call 1: B=16, 2048 of 16384 slots")
    a, b = _call_both(big, W.MLA_SCALE)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    small = W.make_mla_inputs(W.MlaWorkload("mla_small", B=3, cap=700, n_idx=300), seed=22, lens=[0, 150, 700])
    log("[no-alloc] call 2: B=3, 300 of 700 slots, an empty row")
    a, b = _call_both(small, W.MLA_SCALE)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.all(b[0] == 0)
