"""lk_decode_select (the decode step's scores and their per-row top-k from one call) on
the GPU.  Rows of at most 1024 keys run as one launch whose top-k reads the block's
scores from LDS; rows past that run as the two launches.  Either way the result must
equal lk_decode_score + lk_topk bit for bit (scores, indices in the same order, cache,
quantized query and folded weights) and the oracle to the score tolerance, with strict
top-k acceptance on the oracle's scores."""
import numpy as np
import pytest
import torch

from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline_fused, log, tol

pytestmark = pytest.mark.gpu


def _ragged(name, lens, T, k, seed):
    wl = W.Workload(name=name, B=len(lens), S=1, T=T, cap=T + 8, start_pos=-1, k=k, causal=False, ragged=True)
    base = W.make_inputs(wl, seed=seed)
    lt = torch.tensor(lens, dtype=torch.int32)
    return W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))


def _assert_same(two, sel, wl):
    """The one-call result against the two-launch step on the same inputs."""
    assert torch.equal(two.idx.reshape(wl.B, wl.k), sel.idx.reshape(wl.B, wl.k)), "indices differ"
    if sel.scores is not None:
        assert torch.equal(two.scores.reshape(wl.B, wl.T).view(torch.int32),
                           sel.scores.reshape(wl.B, wl.T).view(torch.int32)), "scores differ"
    assert torch.equal(two.q_fp8.reshape(-1), sel.q_fp8.reshape(-1)), "quantized query differs"
    assert torch.equal(two.w_eff.reshape(-1).view(torch.int32), sel.w_eff.reshape(-1).view(torch.int32))
    assert torch.equal(two.cache, sel.cache), "cache bytes differ"
    assert torch.equal(two.cache_scale.view(torch.int32), sel.cache_scale.view(torch.int32)), "cache scales differ"


def _check_oracle(inp, g, rows, rope=False):
    wl = inp.wl
    oc = OracleCase(inp, rope=rope)
    ref = [oc.row(b, 0) for b in rows]
    tau = tol(max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref))
    if g.scores is not None:
        scores = g.scores.cpu().numpy().reshape(wl.B, wl.T)
        compare_scores([scores[b] for b in rows], ref)
    idx = g.idx.cpu().numpy().reshape(wl.B, wl.k)
    for b, r in zip(rows, ref):
        compare_topk(idx[b], r, wl.k, tau)


@pytest.mark.parametrize("rope", [False, True])
def test_stated_decode_step_one_launch(rope):
    """The pages' stated decode step (position 1000: 1001 keys, top-256), one launch."""
    wl = W.WORKLOADS["decode_b1_t1001"]
    inp = W.make_inputs(wl, seed=0)
    log(f"[select] decode_b1_t1001 rope={rope}")
    two = gpu_pipeline_fused(inp, rope=rope)
    sel = gpu_pipeline_fused(inp, rope=rope, select=True)
    _assert_same(two, sel, wl)
    _check_oracle(inp, sel, [0], rope=rope)
    bare = gpu_pipeline_fused(inp, rope=rope, select=True, keep_scores=False)
    assert bare.scores is None
    assert torch.equal(bare.idx, sel.idx), "indices depend on whether the scores are kept"


@pytest.mark.parametrize("k", [1, 256, 1001])
def test_ragged_rows_one_launch(k):
    """Row lengths around k and around the 256-thread top-k's float4 groups, an empty
    row and a one-key row: every row against the oracle and the two-launch step."""
    lens = [0, 1, 2, 3, 4, 5, 31, 32, 33, 255, 256, 257, 700, 1000, 1001]
    inp = _ragged(f"select_ragged_k{k}", lens, T=1001, k=k, seed=11)
    log(f"[select] ragged rows, T=1001, k={k}")
    two = gpu_pipeline_fused(inp)
    sel = gpu_pipeline_fused(inp, select=True)
    _assert_same(two, sel, inp.wl)
    _check_oracle(inp, sel, list(range(inp.wl.B)))


def test_many_rows_full_block():
    """More rows than compute units (300), T = 1024 (the longest one-launch row), RoPE on,
    with and without the scores kept."""
    edge = [0, 1, 17, 255, 256, 511, 512, 513, 1000, 1023, 1024]
    lens = [edge[i % len(edge)] for i in range(300)]
    inp = _ragged("select_many_rows", lens, T=1024, k=512, seed=12)
    log("[select] 300 rows, T=1024, k=512, rope")
    two = gpu_pipeline_fused(inp, rope=True)
    sel = gpu_pipeline_fused(inp, rope=True, select=True)
    _assert_same(two, sel, inp.wl)
    bare = gpu_pipeline_fused(inp, rope=True, select=True, keep_scores=False)
    assert torch.equal(bare.idx, sel.idx)
    rows = sorted(set(range(0, 11)) | {57, 150, 256, 299})
    _check_oracle(inp, sel, rows, rope=True)


@pytest.mark.parametrize("name", ["decode_b16_t16384", "ragged_decode_b64"])
def test_two_launch_rows(name):
    """Rows past one key block take lk_decode_score's launch and lk_topk's: the same bits."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=2)
    log(f"[select] {name} (two launches)")
    two = gpu_pipeline_fused(inp)
    sel = gpu_pipeline_fused(inp, select=True)
    _assert_same(two, sel, wl)


def test_first_row_past_one_block():
    """T = 1025 (the shortest two-launch row) with lengths on both sides of 1024."""
    inp = _ragged("select_t1025", [1, 1023, 1024, 1025, 600], T=1025, k=300, seed=13)
    log("[select] T=1025")
    two = gpu_pipeline_fused(inp)
    sel = gpu_pipeline_fused(inp, select=True)
    _assert_same(two, sel, inp.wl)
    _check_oracle(inp, sel, list(range(inp.wl.B)))


def test_causal_rows():
    """Decode rows with the causal limit inside the row (L = start_pos + 1 < T): the slots
    past it are -inf and out of the selection, in one launch and past one block."""
    for T, k in ((1001, 256), (3000, 700)):
        wl = W.Workload(name=f"select_causal_t{T}", B=3, S=1, T=T, cap=T, start_pos=T // 2, k=k,
                        causal=True, ragged=False)
        inp = W.make_inputs(wl, seed=14)
        log(f"[select] causal rows, T={T}, start_pos={wl.start_pos}, k={k}")
        two = gpu_pipeline_fused(inp)
        sel = gpu_pipeline_fused(inp, select=True)
        _assert_same(two, sel, wl)
        _check_oracle(inp, sel, list(range(wl.B)))
