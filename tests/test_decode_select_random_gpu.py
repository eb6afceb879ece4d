"""lk_decode_select on seeded random shapes around its one-launch limit (1024 keys per
row): ragged row lengths (empty rows and full rows included), k from 1 to T, RoPE on or
off, scores kept or left out (past 1024 keys a call without a score buffer must fail
with LK_E_NULL before any launch; the case then runs with the scores kept).  Every case
must equal lk_decode_score + lk_topk bit for bit (indices in the same order, scores,
cache, quantized query, folded weights), and two rows per case are checked against the
oracle (scores to the tolerance, the oracle's top-k accepted strictly)."""
import numpy as np
import pytest
import torch

from sparse_attention_lightning_fp8_amd import _lib
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline_fused, log, tol

pytestmark = pytest.mark.gpu

# Row counts at and around the one-launch limit and the 256-thread top-k's groups.
T_CHOICES = [1, 2, 3, 63, 64, 65, 255, 256, 257, 700, 1000, 1023, 1024, 1025, 1100, 2048, 3001]


def _case(i):
    rng = np.random.RandomState(1000 + i)
    T = int(T_CHOICES[i % len(T_CHOICES)])
    B = int(rng.randint(1, 9))
    lens = rng.randint(0, T + 1, size=B)
    lens[rng.randint(0, B)] = T                       # one full row in every case
    k = int(rng.choice([1, max(1, T // 3), T, int(rng.randint(1, T + 1))]))
    rope = bool(rng.randint(0, 2))
    keep = bool(rng.randint(0, 2))
    return T, [int(x) for x in lens], k, rope, keep


def _inputs(i, T, lens, k):
    wl = W.Workload(name=f"select_random_{i}", B=len(lens), S=1, T=T, cap=T + 8, start_pos=-1, k=k,
                    causal=False, ragged=True)
    base = W.make_inputs(wl, seed=500 + i)
    lt = torch.tensor(lens, dtype=torch.int32)
    return W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))


@pytest.mark.parametrize("i", range(len(T_CHOICES)))
def test_random_case(i):
    T, lens, k, rope, keep = _case(i)
    inp = _inputs(i, T, lens, k)
    wl = inp.wl
    log(f"[select random {i}] B={wl.B} T={T} k={k} rope={rope} keep_scores={keep} lens={lens}")
    two = gpu_pipeline_fused(inp, rope=rope)
    if not keep and T > 1024:
        with pytest.raises(_lib.LkError) as e:
            gpu_pipeline_fused(inp, rope=rope, select=True, keep_scores=False)
        assert _lib.STATUS_NAMES[e.value.status] == "LK_E_NULL"
        keep = True
    sel = gpu_pipeline_fused(inp, rope=rope, select=True, keep_scores=keep)
    assert torch.equal(two.idx.reshape(wl.B, k), sel.idx.reshape(wl.B, k)), "indices differ"
    if keep:
        assert torch.equal(two.scores.reshape(wl.B, T).view(torch.int32),
                           sel.scores.reshape(wl.B, T).view(torch.int32)), "scores differ"
    elif T <= 1024:
        assert sel.scores is None
    assert torch.equal(two.q_fp8.reshape(-1), sel.q_fp8.reshape(-1)), "quantized query differs"
    assert torch.equal(two.w_eff.reshape(-1).view(torch.int32), sel.w_eff.reshape(-1).view(torch.int32))
    assert torch.equal(two.cache, sel.cache), "cache bytes differ"
    assert torch.equal(two.cache_scale.view(torch.int32), sel.cache_scale.view(torch.int32))
    # two rows against the oracle: the longest and one drawn from the case's seed
    rows = sorted({int(np.argmax(lens)), int(np.random.RandomState(2000 + i).randint(0, wl.B))})
    oc = OracleCase(inp, rope=rope)
    ref = [oc.row(b, 0) for b in rows]
    fin = max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref)
    scores = two.scores.cpu().numpy().reshape(wl.B, T)
    compare_scores([scores[b] for b in rows], ref)
    idx = sel.idx.cpu().numpy().reshape(wl.B, k)
    for b, r in zip(rows, ref):
        compare_topk(idx[b], r, k, tol(fin))
