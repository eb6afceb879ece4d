"""Sparse MLA decode attention (lk_sparse_mla_decode) on the GPU against the oracle
(reading R13).  Tolerance from the arithmetic: logits and softmax in fp32 from exact
bf16 products; p rounded to bf16 (relative error <= 2^-9) for the weighted sum, which
keeps the output a convex combination, so |o - o_ref| <= 2 * 2^-9 * max|c| over the
row's selected latent rows (+ fp32 accumulation, far below)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_rows(inp, out, rows, scale):
    o = out.cpu().numpy()
    for b in rows:
        sel = inp.idx[b].numpy()
        ref = O.sparse_mla_row(W.bf16_bits(inp.q_lat[b]), W.bf16_bits(inp.q_rope[b]), W.bf16_bits(inp.kv_lat[b]),
                               W.bf16_bits(inp.kv_rope[b]), sel, scale)
        valid = sel[(sel >= 0) & (sel < inp.kv_lat.shape[1])]
        vmax = float(np.abs(inp.kv_lat[b][torch.from_numpy(valid).long()].float().numpy()).max()) if valid.size else 0.0
        tau = 2.0 * 2.0 ** -9 * vmax + 1e-6
        err = float(np.max(np.abs(o[b] - ref)))
        assert err <= tau, f"row {b}: max err {err:.3e} > tol {tau:.3e}"
        if valid.size == 0:
            assert np.all(o[b] == 0)


def _run(inp, scale):
    d = lambda t: t.to(DEV)
    out = api.lk_sparse_mla_decode(d(inp.q_lat), d(inp.q_rope), d(inp.kv_lat), d(inp.kv_rope), d(inp.idx), scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("cap,n_idx", [(64, 1), (100, 33), (600, 256), (3000, 300), (4096, 2048)])
def test_mla_small_rows(cap, n_idx):
    wl = W.MlaWorkload(f"mla_{cap}_{n_idx}", B=3, cap=cap, n_idx=n_idx)
    inp = W.make_mla_inputs(wl, seed=cap + n_idx)
    log(f"[mla] cap={cap} n_idx={n_idx}")
    _check_rows(inp, _run(inp, W.MLA_SCALE), range(wl.B), W.MLA_SCALE)


def test_mla_padding_invalid_and_empty_rows():
    wl = W.MlaWorkload("mla_pad", B=4, cap=500, n_idx=300)
    inp = W.make_mla_inputs(wl, seed=11, lens=[0, 1, 45, 500])     # rows padded with -1 past min(n, len)
    idx = inp.idx.clone()
    idx[3, 10] = 500          # outside [0, cap): ignored
    idx[3, 11] = -7           # negative: ignored
    inp.idx = idx
    log("[mla] padding, invalid slots, empty row")
    out = _run(inp, W.MLA_SCALE)
    # the oracle ignores only -1: drop the two invalid entries for it
    idx2 = idx.clone()
    idx2[3, 10] = -1
    idx2[3, 11] = -1
    inp.idx = idx2
    _check_rows(inp, out, range(wl.B), W.MLA_SCALE)


def test_mla_peaked_softmax_and_scales():
    """Large logits (a few keys dominate) and a tiny scale (near-uniform weights)."""
    wl = W.MlaWorkload("mla_peak", B=2, cap=1000, n_idx=512)
    inp = W.make_mla_inputs(wl, seed=12)
    for scale in (0.5, 1e-4):
        log(f"[mla] scale {scale}")
        _check_rows(inp, _run(inp, scale), range(wl.B), scale)


def test_mla_decode_workload_sampled_rows():
    wl = W.MLA_WORKLOADS["mla_decode_b16_t16384"]
    inp = W.make_mla_inputs(wl, seed=0)
    log("[mla] mla_decode_b16_t16384")
    out = _run(inp, W.MLA_SCALE)
    _check_rows(inp, out, [0, 7, 15], W.MLA_SCALE)


def test_mla_deterministic_and_order_free():
    wl = W.MlaWorkload("mla_det", B=2, cap=2048, n_idx=700)
    inp = W.make_mla_inputs(wl, seed=13)
    a = _run(inp, W.MLA_SCALE)
    b = _run(inp, W.MLA_SCALE)
    assert torch.equal(a, b)
