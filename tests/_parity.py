"""Shared parity machinery: the oracle side (CPU, from oracle/ only) and the GPU side
(through the C ABI only), on the same seeded inputs from the workload generator.
No value flows from the GPU side into the oracle side."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import workloads as W


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tol(ref_finite_max: float) -> float:
    """Score tolerance: 1e-5 * max|S_ref| + 1e-6 over the compared finite outputs."""
    return 1e-5 * ref_finite_max + 1e-6


# ------------------------------------------------------------------ oracle side
@dataclass
class OracleRow:
    b: int
    t: int
    L: int
    scores: np.ndarray    # float64 [T]
    topk: np.ndarray      # int32 [k]


class OracleCase:
    """Oracle results for selected query rows of a workload.  With `rope`, every key and
    query row is rotated by RoPE at its absolute position first (key: its cache row;
    query token t of sequence b: positions[b] + t)."""

    def __init__(self, inp: W.Inputs, rope: bool = False):
        self.inp = inp
        self.wl = inp.wl
        self.rope = rope
        self._kq: Dict[int, tuple] = {}

    def keys(self, b: int, n: int):
        """Oracle quantization of cache rows [0, n) of sequence b."""
        got = self._kq.get(b)
        if got is None or got[0].shape[0] < n:
            bits = W.bf16_bits(self.inp.k[b, :n])
            if self.rope:
                c, s = W.rope_tables(np.arange(n))
                codes, scales = O.rope_quantize_rows(bits, c, s)
            else:
                codes, scales = O.quantize_rows(bits)
            self._kq[b] = (codes, scales)
        codes, scales = self._kq[b]
        return codes[:n], scales[:n]

    def query(self, b: int, t: int):
        bits = W.bf16_bits(self.inp.q[b, t])
        if self.rope:
            c, s = W.rope_tables([W.query_positions(self.inp)[b, t]])
            q8, qs = O.rope_quantize_rows(bits, c, s, rows_per_table_row=64)
        else:
            q8, qs = O.quantize_rows(bits)
        w_eff = O.fold_weights(self.inp.w[b, t].numpy(), qs)
        return q8, qs, w_eff

    def row_len(self, b: int, t: int) -> int:
        wl = self.wl
        sl = max(int(self.inp.lens[b]), 0) if self.inp.lens is not None else -1
        return O.valid_len(wl.T, sl, wl.causal, wl.start_pos, t)

    def row(self, b: int, t: int) -> OracleRow:
        wl = self.wl
        L = self.row_len(b, t)
        q8, qs, w_eff = self.query(b, t)
        k8, ks = self.keys(b, max(L, 1))
        k8_full = np.zeros((wl.T, 128), np.uint8)
        ks_full = np.ones(wl.T, np.float32)
        k8_full[:L] = k8[:L]
        ks_full[:L] = ks[:L]
        s = O.score_row(q8, w_eff, k8_full, ks_full, wl.T, L)
        return OracleRow(b, t, L, s, O.topk(s, L, wl.k))


# ------------------------------------------------------------------ GPU side
@dataclass
class GpuResult:
    cache: torch.Tensor
    cache_scale: torch.Tensor
    q_fp8: torch.Tensor
    w_eff: torch.Tensor
    q_scale: torch.Tensor
    scores: torch.Tensor
    idx: torch.Tensor


def _rope_dev(positions, device):
    c, s = W.rope_tables(positions)
    return torch.from_numpy(c).to(device), torch.from_numpy(s).to(device)


def write_prefix(inp: W.Inputs, cache, cache_scale, rope: bool, device="cuda:0", upto=None) -> None:
    """Write cache rows [0, upto[b]) of every sequence (all rows if upto is None),
    rotated by RoPE at their positions when `rope` is set."""
    from sparse_attention_lightning_fp8_amd import api
    wl = inp.wl
    k = inp.k.to(device)
    if upto is None and not rope:
        api.lk_quantize_keys(k, cache, cache_scale, row_offset=0)
        return
    q0 = torch.empty((0, 64, 128), dtype=torch.bfloat16, device=device)
    w0 = torch.empty((0, 64), dtype=torch.float32, device=device)
    for b in range(wl.B):
        n = wl.cap if upto is None else int(upto[b])
        if n <= 0:
            continue
        api.lk_prepare(k[b:b + 1, :n], cache[b:b + 1], cache_scale[b:b + 1], q0, w0,
                       k_rope=_rope_dev(np.arange(n), device) if rope else None)


def gpu_pipeline(inp: W.Inputs, device="cuda:0", rope: bool = False) -> GpuResult:
    """The hot path through the C ABI: cache prefix written first, then one step:
    key write of the step's rows with query quantize + fold (one lk_prepare launch),
    index score, top-k.  With `rope`, keys and queries are rotated by RoPE at their
    positions."""
    from sparse_attention_lightning_fp8_amd import api
    wl = inp.wl
    k = inp.k.to(device)
    cache = torch.zeros((wl.B, wl.cap, 128), dtype=torch.uint8, device=device)
    cache_scale = torch.zeros((wl.B, wl.cap), dtype=torch.float32, device=device)
    positions = inp.positions.to(device)
    # prefix: every cache row, then the step's own rows again through `positions`
    write_prefix(inp, cache, cache_scale, rope, device)
    rows_step = k.new_empty((wl.B, wl.S, 128))
    for b in range(wl.B):
        p0 = int(inp.positions[b])
        rows_step[b] = k[b, p0:p0 + wl.S]
    q = inp.q.to(device)
    w = inp.w.to(device)
    q_scale = torch.empty_like(w)
    qpos = W.query_positions(inp)
    k_rope = _rope_dev(qpos.reshape(-1), device) if rope else None     # the step's keys sit at the query positions
    q_rope = _rope_dev(qpos.reshape(-1), device) if rope else None
    q_fp8, w_eff = api.lk_prepare(rows_step, cache, cache_scale, q, w, positions=positions, q_scale=q_scale,
                                  k_rope=k_rope, q_rope=q_rope)
    seq_len = inp.lens.to(device) if inp.lens is not None else None
    scores = api.lk_index_score(q_fp8, w_eff, cache, cache_scale, wl.T, start_pos=wl.start_pos,
                                seq_len=seq_len, causal=wl.causal)
    idx = api.lk_topk(scores, wl.k, start_pos=wl.start_pos, seq_len=seq_len, causal=wl.causal)
    torch.cuda.synchronize()
    return GpuResult(cache, cache_scale, q_fp8, w_eff, q_scale, scores, idx)


def gpu_pipeline_fused(inp: W.Inputs, device="cuda:0", rope: bool = False, select: bool = False,
                       keep_scores: bool = True) -> GpuResult:
    """The fused decode step through the C ABI: the cache prefix [0, L-1) of each
    sequence is written first (slot L-1 and beyond hold 0xAA garbage), then one
    lk_decode_score launch writes the new key at L-1, quantizes the query and scores,
    then lk_topk.  With `select`, the same step as one lk_decode_select call (scores
    left out when not `keep_scores`).  With `rope`, the prefix keys are rotated at their
    positions and the step's query and new key at position L-1."""
    from sparse_attention_lightning_fp8_amd import api
    wl = inp.wl
    assert wl.S == 1
    k = inp.k.to(device)
    cache = torch.full((wl.B, wl.cap, 128), 0xAA, dtype=torch.uint8, device=device)
    cache_scale = torch.full((wl.B, wl.cap), 3.0, dtype=torch.float32, device=device)
    seq_len = inp.lens.to(device) if inp.lens is not None else None
    new_rows = k.new_empty((wl.B, 128))
    Ls = []
    for b in range(wl.B):
        sl = int(inp.lens[b]) if inp.lens is not None else -1
        L = O.valid_len(wl.T, sl, wl.causal, wl.start_pos, 0)
        Ls.append(L)
        new_rows[b] = k[b, max(L - 1, 0)]
    write_prefix(inp, cache, cache_scale, rope, device, upto=[max(L - 1, 0) for L in Ls])
    # the step's token sits at positions[b] (= L - 1 whenever L >= 1): its table row
    # rotates both the query and the new key
    rope_t = _rope_dev(W.query_positions(inp)[:, 0], device) if rope else None
    q = inp.q.to(device).reshape(wl.B, 64, 128)
    w = inp.w.to(device).reshape(wl.B, 64)
    q_fp8 = torch.empty((wl.B, 1, 64, 128), dtype=torch.uint8, device=device)
    w_eff = torch.empty((wl.B, 1, 64), dtype=torch.float32, device=device)
    if select:
        scores, idx = api.lk_decode_select(q, w, new_rows, cache, cache_scale, wl.T, wl.k, start_pos=wl.start_pos,
                                           seq_len=seq_len, causal=wl.causal, keep_scores=keep_scores,
                                           q_fp8_out=q_fp8, w_eff_out=w_eff, rope=rope_t)
    else:
        scores = api.lk_decode_score(q, w, new_rows, cache, cache_scale, wl.T, start_pos=wl.start_pos,
                                     seq_len=seq_len, causal=wl.causal, q_fp8_out=q_fp8, w_eff_out=w_eff,
                                     rope=rope_t)
        idx = api.lk_topk(scores, wl.k, start_pos=wl.start_pos, seq_len=seq_len, causal=wl.causal)
    torch.cuda.synchronize()
    return GpuResult(cache, cache_scale, q_fp8, w_eff, None, scores, idx)


# ------------------------------------------------------------------ comparisons
def compare_scores(gpu_rows: List[np.ndarray], ref_rows: List[OracleRow]) -> float:
    """Assert the -inf pattern is exact and finite entries agree within tolerance.
    Returns max|err| / max|ref| for reporting."""
    fin_max = max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref_rows)
    tau = tol(fin_max)
    worst = 0.0
    for g, r in zip(gpu_rows, ref_rows):
        ref_inf = np.isneginf(r.scores)
        assert np.array_equal(np.isneginf(g), ref_inf), f"-inf pattern differs in row (b={r.b}, t={r.t})"
        assert np.all(np.isfinite(g[~ref_inf])), f"non-finite score in row (b={r.b}, t={r.t})"
        err = np.max(np.abs(g[~ref_inf].astype(np.float64) - r.scores[~ref_inf]), initial=0.0)
        assert err <= tau, f"row (b={r.b}, t={r.t}): max err {err:.3e} > tol {tau:.3e}"
        worst = max(worst, err)
    return worst / fin_max if fin_max > 0 else 0.0


def compare_topk(gpu_idx: np.ndarray, r: OracleRow, k: int, tau: float) -> None:
    """Top-k acceptance against the oracle's fp64 scores: same size, no duplicates, all
    indices valid, and any disagreement only between keys within tau of the boundary."""
    kr = min(k, r.L)
    g = gpu_idx[:kr]
    assert np.all(gpu_idx[kr:] == -1), "padding must be -1"
    assert len(set(g.tolist())) == kr, "duplicate indices"
    assert np.all((g >= 0) & (g < r.L)), "index outside the valid prefix"
    o = r.topk[:kr]
    if kr == 0:
        return
    vk = np.sort(r.scores[o])[0]          # k-th largest oracle score
    diff = set(g.tolist()) ^ set(o.tolist())
    for i in diff:
        assert abs(r.scores[i] - vk) <= tau, f"row (b={r.b}, t={r.t}): index {i} off the boundary by {r.scores[i] - vk:.3e}"
