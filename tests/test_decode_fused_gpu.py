"""lk_decode_score (new key write + query quantization + index score in one launch)
on the GPU against the oracle: the new key's cache bytes and scale, the quantized
query and folded weights bit-exact, scores within 1e-5 max|S_ref| + 1e-6, top-k sets
equal up to swaps at the k-th boundary; and bitwise equal to the unfused path."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline, gpu_pipeline_fused, log, tol

pytestmark = pytest.mark.gpu
DECODE = ["decode_b1_t1001", "decode_b16_t16384", "ragged_decode_b64"]


def _check_against_oracle(inp, g, rows):
    wl = inp.wl
    oc = OracleCase(inp)
    cache = g.cache.cpu().numpy()
    cscale = g.cache_scale.cpu().numpy()
    q8 = g.q_fp8.cpu().numpy().reshape(wl.B, 64, 128)
    we = g.w_eff.cpu().numpy().reshape(wl.B, 64)
    scores = g.scores.cpu().numpy().reshape(wl.B, wl.T)
    idx = g.idx.cpu().numpy().reshape(wl.B, wl.k)
    ref = []
    for b in rows:
        r = oc.row(b, 0)
        ref.append(r)
        oq8, _, ow = oc.query(b, 0)
        assert np.array_equal(q8[b], oq8), f"query bytes differ (b={b})"
        assert np.array_equal(we[b].view(np.uint32), ow.view(np.uint32)), f"folded weights differ (b={b})"
        if r.L >= 1:
            k8, ks = oc.keys(b, r.L)
            assert np.array_equal(cache[b, r.L - 1], k8[r.L - 1]), f"new key bytes differ (b={b}, slot {r.L - 1})"
            assert cscale[b, r.L - 1] == ks[r.L - 1], f"new key scale differs (b={b})"
        assert np.all(cache[b, max(r.L, 0):] == 0xAA), f"bytes written past slot L-1 (b={b})"
    worst = compare_scores([scores[b] for b in rows], ref)
    tau = tol(max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref))
    for b, r in zip(rows, ref):
        compare_topk(idx[b], r, wl.k, tau)
    return worst


@pytest.mark.parametrize("name", DECODE)
def test_fused_decode_workloads(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    log(f"[fused] {name}: B={wl.B} T={wl.T}")
    g = gpu_pipeline_fused(inp)
    if inp.lens is not None:
        lens = inp.lens.numpy()
        rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 63})
    else:
        rows = sorted({0, wl.B // 2, wl.B - 1})
    worst = _check_against_oracle(inp, g, rows)
    log(f"[fused] {name}: worst relative score error {worst:.2e}")


@pytest.mark.parametrize("name", DECODE)
def test_fused_equals_unfused(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=1)
    log(f"[fused] {name} vs lk_prepare + lk_index_score")
    a = gpu_pipeline(inp)
    f = gpu_pipeline_fused(inp)
    sa = a.scores.reshape(wl.B, wl.T)
    sf = f.scores.reshape(wl.B, wl.T)
    assert torch.equal(sa.view(torch.int32), sf.view(torch.int32))
    assert torch.equal(a.q_fp8.reshape(-1), f.q_fp8.reshape(-1))
    assert torch.equal(a.w_eff.reshape(-1).view(torch.int32), f.w_eff.reshape(-1).view(torch.int32))
    assert torch.equal(a.idx.reshape(wl.B, wl.k), f.idx.reshape(wl.B, wl.k))
    for b in range(wl.B):
        sl = int(inp.lens[b]) if inp.lens is not None else -1
        L = O.valid_len(wl.T, sl, wl.causal, wl.start_pos, 0)
        assert torch.equal(a.cache[b, :L], f.cache[b, :L])
        assert torch.equal(a.cache_scale[b, :L], f.cache_scale[b, :L])


def test_fused_ragged_edges():
    """Row lengths at and around the 1024-key block boundary, a single key, no key,
    and T not a multiple of the block: every row checked whole against the oracle."""
    lens = [0, 1, 2, 31, 32, 33, 1023, 1024, 1025, 2047, 2500, 2600]
    wl = W.Workload(name="ragged_edges", B=len(lens), S=1, T=2600, cap=2700, start_pos=-1, k=2048,
                    causal=False, ragged=True)
    base = W.make_inputs(wl, seed=3)
    lt = torch.tensor(lens, dtype=torch.int32)
    inp = W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))
    log("[fused] ragged edge rows")
    g = gpu_pipeline_fused(inp)
    _check_against_oracle(inp, g, list(range(wl.B)))
