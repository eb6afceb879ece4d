"""Index score + mask on the GPU against the oracle (tolerance 1e-5 max|S_ref| + 1e-6),
plus the invariants that hold bit for bit."""
import zlib

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from tests._parity import log, tol

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quantized_inputs(seed, B, S, cap, wide=False):
    """Oracle-quantized q/k (bf16 N(0,1) draws) and folded weights, as numpy."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, 64, 128, generator=g)
    k = torch.randn(B, cap, 128, generator=g)
    if wide:
        k = k * torch.exp2(torch.randint(-12, 12, (B, cap, 1), generator=g).float())
    w = torch.randn(B, S, 64, generator=g) * 0.125
    qb = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = k.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q8, qs = O.quantize_rows(qb)
    k8, ks = O.quantize_rows(kb)
    w_eff = O.fold_weights(w.numpy().reshape(-1), qs.reshape(-1)).reshape(B, S, 64)
    return q8, w_eff, k8, ks


def _oracle_scores(q8, w_eff, k8, ks, T, start_pos, lens, causal):
    B, S = q8.shape[:2]
    out = np.empty((B, S, T))
    Ls = np.empty((B, S), np.int64)
    for b in range(B):
        for t in range(S):
            sl = max(int(lens[b]), 0) if lens is not None else -1  # the ABI clamps lengths at 0
            L = O.valid_len(T, sl, causal, start_pos, t)
            Ls[b, t] = L
            out[b, t] = O.score_row(q8[b, t], w_eff[b, t], k8[b], ks[b], T, L)
    return out, Ls


def _gpu_scores(q8, w_eff, k8, ks, T, start_pos, lens, causal, stride_pad=0):
    B, cap = k8.shape[:2]
    kc = torch.zeros((B, cap + stride_pad, 128), dtype=torch.uint8, device=DEV)
    kcs = torch.zeros((B, cap + stride_pad), dtype=torch.float32, device=DEV)
    kc[:, :cap] = torch.from_numpy(k8).to(DEV)
    kcs[:, :cap] = torch.from_numpy(ks).to(DEV)
    seq_len = torch.from_numpy(np.asarray(lens, np.int32)).to(DEV) if lens is not None else None
    s = api.lk_index_score(torch.from_numpy(q8).to(DEV), torch.from_numpy(w_eff).to(DEV),
                           kc[:, :cap], kcs[:, :cap], T, start_pos=start_pos, seq_len=seq_len, causal=causal)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def _check(gs, os_):
    fin = np.isfinite(os_)
    assert np.array_equal(np.isneginf(gs), ~fin), "-inf pattern differs"
    m = np.max(np.abs(os_[fin]), initial=0.0)
    err = np.max(np.abs(gs[fin] - os_[fin]), initial=0.0)
    assert err <= tol(m), f"max err {err:.3e} > tol {tol(m):.3e} (max|S| {m:.3e})"
    return err / m if m else 0.0


CASES = [
    # name, B, S, cap, T, start_pos, lens, causal
    ("decode_T1", 1, 1, 8, 1, 0, None, False),
    ("decode_T33", 2, 1, 40, 33, 0, None, False),
    ("decode_T1001", 1, 1, 1001, 1001, 1000, None, False),
    ("decode_T1536_B3", 3, 1, 1600, 1536, 0, None, False),
    ("ragged_edges", 6, 1, 700, 700, 0, [0, 1, 31, 699, 700, 5000], False),
    ("ragged_negative_len", 2, 1, 64, 64, 0, [-3, 64], False),
    ("decode_causal_start", 2, 1, 300, 300, 150, None, True),
    ("prefill_S2", 1, 2, 70, 70, 68, None, True),
    ("prefill_S9_causal", 2, 9, 300, 300, 0, None, True),
    ("prefill_S17_start", 1, 17, 600, 600, 500, None, True),
    ("prefill_noncausal", 1, 12, 513, 513, 0, None, False),
    ("prefill_ragged_causal", 2, 10, 400, 400, 300, [350, 5], True),
    ("prefill_S64_T777", 1, 64, 777, 777, 713, None, True),
]


@pytest.mark.parametrize("name,B,S,cap,T,start_pos,lens,causal", CASES, ids=[c[0] for c in CASES])
def test_score_matches_oracle(name, B, S, cap, T, start_pos, lens, causal):
    q8, w_eff, k8, ks = _quantized_inputs(zlib.crc32(name.encode()) % 1000, B, S, cap)
    log(f"[score] {name}: B={B} S={S} T={T} cap={cap} start={start_pos} causal={causal}")
    gs = _gpu_scores(q8, w_eff, k8, ks, T, start_pos, lens, causal, stride_pad=3)
    os_, _ = _oracle_scores(q8, w_eff, k8, ks, T, start_pos, lens, causal)
    _check(gs, os_)


def test_score_wide_key_scales():
    """Keys spread over 2^-12..2^12 (one power-of-two scale each)."""
    q8, w_eff, k8, ks = _quantized_inputs(7, 2, 1, 1000, wide=True)
    log("[score] wide key scales")
    gs = _gpu_scores(q8, w_eff, k8, ks, 1000, 0, None, False)
    os_, _ = _oracle_scores(q8, w_eff, k8, ks, 1000, 0, None, False)
    _check(gs, os_)


def test_score_random_codes():
    """Uniformly random finite e4m3fn bytes (values 2^-9..448 of both signs)."""
    rng = np.random.default_rng(8)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q8 = rng.choice(codes, (2, 3, 64, 128))
    k8 = rng.choice(codes, (2, 500, 128))
    ks = np.exp2(rng.integers(-20, 0, (2, 500))).astype(np.float32)
    w_eff = (rng.standard_normal((2, 3, 64)) * 1e-4).astype(np.float32)
    log("[score] random codes")
    gs = _gpu_scores(q8, w_eff, k8, ks, 500, 0, None, False)
    os_, _ = _oracle_scores(q8, w_eff, k8, ks, 500, 0, None, False)
    _check(gs, os_)


@pytest.mark.parametrize("S", [1, 8])
def test_score_invariants_bitwise(S):
    """Key permutation permutes columns, 2^j key scales scale columns, w >= 0 gives
    S >= 0, and two runs agree bit for bit."""
    q8, w_eff, k8, ks = _quantized_inputs(9 + S, 1, S, 640)
    T = 640
    log(f"[score] invariants S={S}")
    s0 = _gpu_scores(q8, w_eff, k8, ks, T, 0, None, False)
    s0b = _gpu_scores(q8, w_eff, k8, ks, T, 0, None, False)
    assert np.array_equal(s0.view(np.uint32), s0b.view(np.uint32))
    perm = np.random.default_rng(3).permutation(T)
    s1 = _gpu_scores(q8, w_eff, k8[:, perm], ks[:, perm], T, 0, None, False)
    assert np.array_equal(s1.view(np.uint32), s0[..., perm].view(np.uint32))
    ks2 = ks.copy()
    ks2[:, ::5] *= np.float32(2.0**-7)
    s2 = _gpu_scores(q8, w_eff, k8, ks2, T, 0, None, False)
    assert np.array_equal(s2[..., ::5], s0[..., ::5] * np.float32(2.0**-7))
    s3 = _gpu_scores(q8, np.abs(w_eff), k8, ks, T, 0, None, False)
    assert np.all(s3 >= 0)


def test_score_whole_row_items():
    """Prefill with enough 8-token groups (B * ceil(S / 8) >= 2 x the compute units of an
    MI355X) that each block takes its group's whole key range: ragged lengths, causal
    from start_pos 6000, a partial last token group and T not a multiple of 256.  Every
    row's -inf pattern is checked against the oracle's valid length, and sampled rows
    (both sequences, each side of the length and 8-token group edges) element by element."""
    B, S, T, start_pos, lens = 2, 2053, 9000, 6000, [8000, 9000]
    assert B * ((S + 7) // 8) >= 2 * 256
    q8, w_eff, k8, ks = _quantized_inputs(31, B, S, T)
    log(f"[score] whole-row items: B={B} S={S} T={T} start={start_pos} lens={lens}")
    gs = _gpu_scores(q8, w_eff, k8, ks, T, start_pos, lens, True, stride_pad=5)
    for b in range(B):
        for t in range(S):
            L = O.valid_len(T, lens[b], True, start_pos, t)
            row = gs[b, t]
            assert np.all(np.isfinite(row[:L])) and np.all(np.isneginf(row[L:])), (b, t, L)
    samples = [0, 1, 7, 8, 1998, 1999, 2000, 2047, 2048, 2052]
    errs = []
    for b in range(B):
        for t in samples:
            L = O.valid_len(T, lens[b], True, start_pos, t)
            ref = O.score_row(q8[b, t], w_eff[b, t], k8[b], ks[b], T, L)
            errs.append(_check(gs[b, t][None], ref[None]))
    log(f"[score] whole-row items: max rel err {max(errs):.2e} over {len(errs)} rows")


def _random_code_inputs(rng, B, S, cap):
    """Uniform finite e4m3fn codes for queries and keys, power-of-two key scales and
    small folded weights (the score kernel's input contract, without the quantizer)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q8 = rng.choice(codes, (B, S, 64, 128))
    k8 = rng.choice(codes, (B, cap, 128))
    ks = np.exp2(rng.integers(-12, 0, (B, cap))).astype(np.float32)
    w_eff = (rng.standard_normal((B, S, 64)) * 1e-3).astype(np.float32)
    return q8, w_eff, k8, ks


# Prefill grids on both sides of the whole-row threshold (B * ceil(S / 8) >= 2 x 256
# compute units): 513, 511, 512 and 516 token groups, and a small S; T off the 64- and
# 256-key grids; causal rows from start_pos; ragged lengths 0, 1, inside and past T.
GRID_CASES = [
    # name, B, S, T, start_pos, lens, causal
    ("groups513_causal", 1, 4099, 6000, 1901, None, True),
    ("groups511_causal", 1, 4088, 6000, 1912, None, True),
    ("groups512_ragged", 2, 4096 // 2, 4353, 0, [0, 5000], False),
    ("groups516_ragged_causal", 3, 1370, 5001, 3631, [1, 4999, 5001], True),
    ("small_S_causal", 2, 9, 5000, 4991, None, True),
]


@pytest.mark.parametrize("name,B,S,T,start_pos,lens,causal", GRID_CASES, ids=[c[0] for c in GRID_CASES])
def test_prefill_grid_forms(name, B, S, T, start_pos, lens, causal):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q8, w_eff, k8, ks = _random_code_inputs(rng, B, S, T)
    log(f"[score] prefill grid {name}: B={B} S={S} T={T} start={start_pos} lens={lens} causal={causal}")
    gs = _gpu_scores(q8, w_eff, k8, ks, T, start_pos, lens, causal, stride_pad=7)
    Ls = np.empty((B, S), np.int64)
    for b in range(B):
        sl = max(int(lens[b]), 0) if lens is not None else -1
        for t in range(S):
            L = O.valid_len(T, sl, causal, start_pos, t)
            Ls[b, t] = L
            row = gs[b, t]
            assert np.all(np.isfinite(row[:L])) and np.all(np.isneginf(row[L:])), (b, t, L)
    # rows at the edges of 8-token groups, the first and last, and a few at random
    cand = {0, 7, 8, S // 2, S - 1} | set(int(x) for x in rng.integers(0, S, 3))
    errs = []
    for b in range(B):
        for t in sorted(c for c in cand if 0 <= c < S):
            ref = O.score_row(q8[b, t], w_eff[b, t], k8[b], ks[b], T, int(Ls[b, t]))
            errs.append(_check(gs[b, t][None], ref[None]))
    log(f"[score] prefill grid {name}: max rel err {max(errs):.2e} over {len(errs)} rows")
