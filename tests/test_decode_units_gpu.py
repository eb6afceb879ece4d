"""lk_decode_score when the rows' 1024-key items outnumber one wave of blocks: the fused
step then runs as balanced runs of 512-key units (decode_units_kernel), each block
deriving the same schedule from the row lengths.  Cases aimed at that schedule: empty
rows and rows around the unit and item edges, T not a multiple of 512, more rows than
compute units, long rows among short ones (the cap search), causal limits, RoPE.
Checked against the oracle on chosen rows (scores to the tolerance, strict top-k acceptance, the quantized
query and folded weights, the new key's bytes and scale, nothing written past slot L-1)
and, where every row has a key, bit for bit against the unfused lk_prepare +
lk_index_score + lk_topk."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline, gpu_pipeline_fused, log, tol

pytestmark = pytest.mark.gpu


def _inputs(name, lens, T, k, seed, causal=False, start_pos=-1):
    wl = W.Workload(name=name, B=len(lens), S=1, T=T, cap=T + 8, start_pos=start_pos, k=k, causal=causal,
                    ragged=True)
    base = W.make_inputs(wl, seed=seed)
    lt = torch.tensor(lens, dtype=torch.int32)
    return W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))


def _units_path(wl):
    """Whether lk_decode_score takes the unit runs for this shape on a 256-CU part."""
    nblk = (wl.T + 1023) // 1024
    return wl.B <= 512 and nblk * wl.B * 4 > 256 * 5


def _check(inp, g, rows, rope=False):
    wl = inp.wl
    oc = OracleCase(inp, rope=rope)
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
            assert np.array_equal(cache[b, r.L - 1], k8[r.L - 1]), f"new key bytes differ (b={b})"
            assert cscale[b, r.L - 1] == ks[r.L - 1], f"new key scale differs (b={b})"
        assert np.all(cache[b, max(r.L, 0):] == 0xAA), f"bytes written past slot L-1 (b={b})"
    compare_scores([scores[b] for b in rows], ref)
    tau = tol(max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref))
    for b, r in zip(rows, ref):
        compare_topk(idx[b], r, wl.k, tau)
    # every row: -inf exactly past its valid prefix, finite before it
    for b in range(wl.B):
        sl = int(inp.lens[b]) if inp.lens is not None else -1
        L = O.valid_len(wl.T, sl, wl.causal, wl.start_pos, 0)
        assert np.all(np.isneginf(scores[b, L:])) and np.all(np.isfinite(scores[b, :L])), f"mask (b={b})"


def _same_as_unfused(inp, f):
    wl = inp.wl
    a = gpu_pipeline(inp)
    assert torch.equal(a.scores.reshape(wl.B, wl.T).view(torch.int32), f.scores.reshape(wl.B, wl.T).view(torch.int32))
    assert torch.equal(a.idx.reshape(wl.B, wl.k), f.idx.reshape(wl.B, wl.k))
    assert torch.equal(a.q_fp8.reshape(-1), f.q_fp8.reshape(-1))
    assert torch.equal(a.w_eff.reshape(-1).view(torch.int32), f.w_eff.reshape(-1).view(torch.int32))


def test_unit_and_item_edges():
    """40 rows of up to 16,000 keys (T not a multiple of 512): empty rows, one key, both
    sides of 512 and 1024, the full row, and seeded lengths; every row against the oracle."""
    edges = [0, 1, 2, 511, 512, 513, 1023, 1024, 1025, 1536, 8191, 8192, 15999, 16000]
    rng = np.random.RandomState(21)
    lens = edges + [int(x) for x in rng.randint(1, 16001, size=40 - len(edges))]
    inp = _inputs("units_edges", lens, T=16000, k=700, seed=21)
    assert _units_path(inp.wl)
    log(f"[units] 40 rows, T=16000, lens {lens[:14]} + seeded")
    g = gpu_pipeline_fused(inp)
    _check(inp, g, list(range(inp.wl.B)))


def test_more_rows_than_compute_units():
    """300 rows of up to 2048 keys (the grid is one block per row), empty rows among them;
    every 7th row and the edges against the oracle, every row's mask checked."""
    rng = np.random.RandomState(22)
    lens = [int(x) for x in rng.randint(0, 2049, size=300)]
    lens[:6] = [0, 1, 512, 513, 2047, 2048]
    inp = _inputs("units_300_rows", lens, T=2048, k=300, seed=22)
    assert _units_path(inp.wl)
    log("[units] 300 rows, T=2048")
    g = gpu_pipeline_fused(inp)
    _check(inp, g, sorted(set(range(0, 300, 7)) | set(range(6))))


def test_long_rows_among_short_ones():
    """Sixteen rows of 15,000-16,384 keys among 48 of at most 600: 559 units, so the cap
    search steps past its lower bound (cap 3); bit for bit against the unfused path,
    and the long rows, the shortest and every 6th row against the oracle."""
    rng = np.random.RandomState(23)
    lens = [16384] + [int(x) for x in rng.randint(15000, 16385, size=15)] + [int(x) for x in rng.randint(1, 601, size=48)]
    inp = _inputs("units_long_rows", lens, T=16384, k=2048, seed=23)
    assert _units_path(inp.wl)
    log("[units] 16 long rows among 48 short ones")
    g = gpu_pipeline_fused(inp)
    short = int(np.argmin(lens))
    _check(inp, g, sorted({0, 5, 15, short} | set(range(16, 64, 6))))
    _same_as_unfused(inp, g)


def test_causal_rows():
    """24 rows of T = 16384 with the causal limit at start_pos 9000 (L = 9001 < T)."""
    wl = W.Workload(name="units_causal", B=24, S=1, T=16384, cap=16384, start_pos=9000, k=2048, causal=True,
                    ragged=False)
    inp = W.make_inputs(wl, seed=24)
    assert _units_path(wl)
    log("[units] 24 causal rows, T=16384, start_pos=9000")
    g = gpu_pipeline_fused(inp)
    _check(inp, g, [0, 11, 23])
    _same_as_unfused(inp, g)


def test_ragged_rows_with_rope():
    """The 64-row ragged decode with RoPE on: the rotated query and new key of every
    row's step token, against the oracle on the shortest, longest and every 8th row."""
    wl = W.WORKLOADS["ragged_decode_b64"]
    inp = W.make_inputs(wl, seed=25)
    assert _units_path(wl)
    log("[units] ragged_decode_b64 with RoPE")
    g = gpu_pipeline_fused(inp, rope=True)
    order = np.argsort(inp.lens.numpy(), kind="stable")
    rows = sorted({int(order[0]), int(order[-1])} | set(range(0, wl.B, 8)))
    _check(inp, g, rows, rope=True)
