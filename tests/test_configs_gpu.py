"""The five indexer workloads end to end on the GPU (key write, query quantize and fold,
index score, top-k, in the launch configuration the benchmark times), checked against
the oracle on sampled rows: key and query bytes bit-exact, scores within
1e-5 max|S_ref| + 1e-6, top-k sets equal up to swaps at the k-th boundary, and
lk_topk exactly equal to the oracle's sort on the oracle's own float32 scores."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline, log, tol

pytestmark = pytest.mark.gpu

# (workload, rows to check as (b, t)).  Prefill rows cover every position of an 8-token
# block (the prefill kernel's token group), both sides of 256-key chunk edges (and of
# 128-key half-chunk edges), of 2048/4096-key slice edges, rows whose causal diagonal ends
# mid-chunk, and a spread over token groups.
def _prefill_rows(S, seqs, extra, group_step):
    ts = set(range(8)) | set(range(S - 8, S)) | set(extra)
    ts |= {8 * g + g % 8 for g in range(0, S // 8, group_step)}
    return [(b, t) for b in seqs for t in sorted(x for x in ts if 0 <= x < S)]


SAMPLES = {
    "decode_b1_t1001": [(0, 0)],
    "decode_b16_t16384": [(b, 0) for b in range(16)],
    "ragged_decode_b64": "ragged",
    # causal 4096 x 4096: row t has t + 1 keys
    "prefill_s4096": _prefill_rows(4096, [0], [126, 127, 128, 129, 255, 256, 511, 512, 1000, 2046, 2047,
                                                2048, 2049, 3001, 4094], 11),
    # 4096 new tokens at 12288..16383: row t has 12289 + t keys; slice edges at keys
    # 4096, 8192, 12288; 256-key aligned lengths at t = 255, 2047, 3839, 128-key aligned
    # at t = 127, 3967
    "chunked_prefill_b2_s4096": _prefill_rows(4096, [0, 1], [126, 127, 128, 254, 255, 256, 1023, 2046, 2047,
                                                              2048, 3839, 3840, 3967], 23),
}


def _rows_for(name, inp):
    s = SAMPLES[name]
    if s == "ragged":                                  # every row, the shortest and longest included
        return [(b, 0) for b in range(inp.wl.B)]
    return s


def test_sample_sizes():
    """At least 64 oracle rows for each prefill workload and every decode row of B16."""
    assert len(SAMPLES["prefill_s4096"]) >= 64
    assert len(SAMPLES["chunked_prefill_b2_s4096"]) >= 64
    assert len({b for b, _ in SAMPLES["chunked_prefill_b2_s4096"]}) == 2


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_end_to_end(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    log(f"[config] {name}: B={wl.B} S={wl.S} T={wl.T} k={wl.k}")
    g = gpu_pipeline(inp)
    oc = OracleCase(inp)
    rows = _rows_for(name, inp)
    cache = g.cache.cpu().numpy()
    cscale = g.cache_scale.cpu().numpy()
    q8 = g.q_fp8.cpu().numpy()
    qs = g.q_scale.cpu().numpy()
    we = g.w_eff.cpu().numpy()
    scores = g.scores.cpu().numpy()
    idx = g.idx.cpu().numpy()
    for b in sorted({b for b, _ in rows}):          # quantize each sequence's keys once
        oc.keys(b, max(max(oc.row_len(bb, t) for bb, t in rows if bb == b), 1))
    ref = []
    for (b, t) in rows:
        r = oc.row(b, t)
        ref.append(r)
        # key bytes of every row the oracle quantized for this sequence, and this query
        k8, ks = oc.keys(b, max(r.L, 1))
        n = min(r.L, k8.shape[0])
        assert np.array_equal(cache[b, :n], k8[:n]), f"key bytes differ (b={b})"
        assert np.array_equal(cscale[b, :n].view(np.uint32), ks[:n].view(np.uint32)), f"key scales differ (b={b})"
        oq8, oqs, owe = oc.query(b, t)
        assert np.array_equal(q8[b, t], oq8), f"query bytes differ ({b},{t})"
        assert np.array_equal(qs[b, t].view(np.uint32), oqs.view(np.uint32))
        assert np.array_equal(we[b, t].view(np.uint32), owe.view(np.uint32)), f"w_eff differs ({b},{t})"
    rel = compare_scores([scores[b, t] for (b, t) in rows], ref)
    fin_max = max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref)
    for (b, t), r in zip(rows, ref):
        compare_topk(idx[b, t], r, wl.k, tol(fin_max))
    log(f"[config] {name}: worst |S - S_ref| / max|S_ref| = {rel:.3e}")
    # strict top-k: the GPU selection on the oracle's float32 scores equals the oracle's
    o32 = np.stack([r.scores.astype(np.float32) for r in ref])[:, None, :]
    lens = torch.tensor([r.L for r in ref], dtype=torch.int32, device="cuda:0")
    gi = api.lk_topk(torch.from_numpy(np.ascontiguousarray(o32)).to("cuda:0"), wl.k, seq_len=lens).cpu().numpy()
    for j, r in enumerate(ref):
        want = O.topk(o32[j, 0], r.L, wl.k)
        assert sorted(gi[j, 0].tolist()) == sorted(want.tolist()), f"strict top-k differs ({r.b},{r.t})"
    # every row of the GPU output satisfies the mask and top-k structure
    B, S, T = scores.shape
    for b in range(B):
        for t in range(0, S, 1 if S <= 64 else 3):
            L = oc.row_len(b, t)
            assert np.all(np.isneginf(scores[b, t, L:])) and np.all(np.isfinite(scores[b, t, :L]))
            kr = min(wl.k, L)
            sel = idx[b, t, :kr]
            assert np.all(idx[b, t, kr:] == -1) and np.all((sel >= 0) & (sel < L))
            assert len(np.unique(sel)) == kr
            if kr and kr < L:
                thr = scores[b, t, sel].min()
                assert np.sum(scores[b, t, :L] > thr) < kr
