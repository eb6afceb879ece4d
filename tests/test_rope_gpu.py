"""RoPE in the key write and query preparation on the GPU (reading R12), against the
oracle: bit-exact codes and scales through lk_prepare's tables, and the fused decode
step (lk_decode_score with tables) and the separate path end to end with RoPE on every
key and query."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import (OracleCase, compare_scores, compare_topk, gpu_pipeline, gpu_pipeline_fused, log,
                           tol)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tables(rng, n, mode):
    if mode == "random":
        ang = rng.uniform(-np.pi, np.pi, (n, 32))
        return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    if mode == "positions":
        return W.rope_tables(rng.integers(0, 16384, n))
    if mode == "quarter":
        return np.zeros((n, 32), np.float32), np.ones((n, 32), np.float32)
    if mode == "wide":                                   # |cos|, |sin| up to 4: no unit-norm assumption
        return (rng.uniform(-4, 4, (n, 32)).astype(np.float32), rng.uniform(-4, 4, (n, 32)).astype(np.float32))
    raise ValueError(mode)


@pytest.mark.parametrize("mode", ["random", "positions", "quarter", "wide"])
def test_prepare_rope_bit_exact(mode):
    rng = np.random.default_rng(hash(mode) % 1000)
    g = torch.Generator().manual_seed(40)
    n_seq, n_rows, cap = 3, 37, 64
    x = (torch.randn(n_seq, n_rows, 128, generator=g) *
         torch.exp2(torch.randint(-12, 12, (n_seq, n_rows, 1), generator=g).float())).to(torch.bfloat16)
    n_tok = 29
    q = (torch.randn(n_tok, 64, 128, generator=g) *
         torch.exp2(torch.randint(-12, 12, (n_tok, 64, 1), generator=g).float())).to(torch.bfloat16)
    w = torch.randn(n_tok, 64, generator=g) * 0.125
    kc, ks = _tables(rng, n_seq * n_rows, mode)
    qc, qs_ = _tables(rng, n_tok, mode)
    cache = torch.zeros(n_seq, cap, 128, dtype=torch.uint8, device=DEV)
    cscale = torch.zeros(n_seq, cap, device=DEV)
    qscale = torch.empty(n_tok, 64, device=DEV)
    log(f"[rope] lk_prepare with tables ({mode})")
    q8, we = api.lk_prepare(x.to(DEV), cache, cscale, q.to(DEV), w.to(DEV), row_offset=5, q_scale=qscale,
                            k_rope=(torch.from_numpy(kc).to(DEV), torch.from_numpy(ks).to(DEV)),
                            q_rope=(torch.from_numpy(qc).to(DEV), torch.from_numpy(qs_).to(DEV)))
    torch.cuda.synchronize()
    ok, os_ = O.rope_quantize_rows(W.bf16_bits(x).reshape(-1, 128), kc, ks)
    got = cache[:, 5:5 + n_rows].cpu().numpy().reshape(-1, 128)
    assert np.array_equal(got, ok)
    assert np.array_equal(cscale[:, 5:5 + n_rows].cpu().numpy().reshape(-1).view(np.uint32), os_.view(np.uint32))
    oq, oqs = O.rope_quantize_rows(W.bf16_bits(q).reshape(-1, 128), qc, qs_, rows_per_table_row=64)
    assert np.array_equal(q8.cpu().numpy().reshape(-1, 128), oq)
    assert np.array_equal(qscale.cpu().numpy().reshape(-1).view(np.uint32), oqs.view(np.uint32))
    ow = O.fold_weights(w.numpy().reshape(-1), oqs)
    assert np.array_equal(we.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32))


def _check(inp, g, rows, rope=True):
    wl = inp.wl
    oc = OracleCase(inp, rope=rope)
    scores = g.scores.cpu().numpy().reshape(wl.B * wl.S, wl.T)
    idx = g.idx.cpu().numpy().reshape(wl.B * wl.S, wl.k)
    q8 = g.q_fp8.cpu().numpy().reshape(wl.B, wl.S, 64, 128)
    cache = g.cache.cpu().numpy()
    ref = []
    for (b, t) in rows:
        r = oc.row(b, t)
        ref.append(r)
        oq8, _, _ = oc.query(b, t)
        assert np.array_equal(q8[b, t], oq8), f"query bytes (b={b}, t={t})"
        k8, _ = oc.keys(b, max(r.L, 1))
        assert np.array_equal(cache[b, :r.L], k8[:r.L]), f"key bytes (b={b})"
    compare_scores([scores[b * wl.S + t] for b, t in rows], ref)
    tau = tol(max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref))
    for (b, t), r in zip(rows, ref):
        compare_topk(idx[b * wl.S + t], r, wl.k, tau)


@pytest.mark.parametrize("name", ["decode_b1_t1001", "decode_b16_t16384", "ragged_decode_b64"])
def test_fused_decode_with_rope(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=5)
    log(f"[rope] fused decode {name}")
    g = gpu_pipeline_fused(inp, rope=True)
    rows = [(0, 0), (wl.B - 1, 0)] if wl.B > 1 else [(0, 0)]
    _check(inp, g, rows)


@pytest.mark.parametrize("name", ["decode_b1_t1001", "prefill_s4096"])
def test_separate_path_with_rope(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=6)
    log(f"[rope] separate path {name}")
    g = gpu_pipeline(inp, rope=True)
    rows = [(0, 0)] if wl.S == 1 else [(0, t) for t in (0, 5, 2047, 4095)]
    _check(inp, g, rows)
