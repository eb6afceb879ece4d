"""Per-row top-k on the GPU: exactly the oracle's set on the same float32 scores."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from tests._parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_topk(scores: np.ndarray, k: int, lens=None, causal=False, start_pos=0):
    s = torch.from_numpy(np.ascontiguousarray(scores, np.float32)).to(DEV)
    sl = torch.from_numpy(np.asarray(lens, np.int32)).to(DEV) if lens is not None else None
    idx = api.lk_topk(s, k, start_pos=start_pos, seq_len=sl, causal=causal)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _check_exact(scores, k, gidx, lens=None, causal=False, start_pos=0):
    B, S, T = scores.shape
    for b in range(B):
        for t in range(S):
            sl = max(int(lens[b]), 0) if lens is not None else -1
            L = O.valid_len(T, sl, causal, start_pos, t)
            want = O.topk(np.ascontiguousarray(scores[b, t], np.float32), L, k)
            got = gidx[b, t]
            assert sorted(got.tolist()) == sorted(want.tolist()), f"row ({b},{t}) L={L}"


@pytest.mark.parametrize("T,k", [(1, 1), (5, 2), (1001, 256), (2049, 2048), (4096, 2048), (16384, 2048),
                                 (16384, 1), (16384, 16384), (3000, 3000)])
def test_topk_random_rows_exact(T, k):
    rng = np.random.default_rng(T + k)
    scores = rng.standard_normal((2, 3, T)).astype(np.float32)
    log(f"[topk] random T={T} k={k}")
    _check_exact(scores, k, _gpu_topk(scores, k), None)


@pytest.mark.parametrize("T", [5000, 3000])          # the 1024- and the 256-thread kernel
def test_topk_ties_signed_zeros_and_infinities(T):
    rng = np.random.default_rng(5)
    s = rng.integers(-4, 4, (3, 2, T)).astype(np.float32)      # heavy ties
    s[0, 0, ::2] = -0.0
    s[0, 0, 1::2] = 0.0
    s[1, 1, :] = -np.inf
    s[1, 1, 17] = 1.0
    s[2, 0, :] = 3.0                                           # all equal
    s[2, 1, 100:] = -np.inf
    log(f"[topk] ties T={T}")
    for k in (1, 7, 2048, T - 1):
        _check_exact(s, k, _gpu_topk(s, k), None)


def test_topk_ragged_and_causal_rows():
    rng = np.random.default_rng(6)
    T = 3000
    s = rng.standard_normal((4, 1, T)).astype(np.float32)
    lens = [0, 1, 2048, 2500]
    log("[topk] ragged")
    _check_exact(s, 2048, _gpu_topk(s, 2048, lens=lens), lens=lens)
    s2 = rng.standard_normal((2, 40, 2100)).astype(np.float32)
    log("[topk] causal")
    g = _gpu_topk(s2, 2048, causal=True, start_pos=2040)
    _check_exact(s2, 2048, g, causal=True, start_pos=2040)


def _rank_ordered(r, v):
    """Scores non-increasing, and indices ascending among equal scores."""
    dv = np.diff(v)
    return bool(np.all(dv <= 0) and np.all((dv < 0) | (np.diff(r) > 0)))


def test_topk_deterministic_and_ordered():
    rng = np.random.default_rng(7)
    ints = rng.integers(0, 50, (2, 16384)).astype(np.float32)     # ties: the cut bin is one value
    normal = rng.standard_normal((2, 16384)).astype(np.float32)   # a few distinct values at the cut
    s = np.stack([ints, normal])                                  # [2 sequences, 2 rows, 16384]
    log("[topk] determinism")
    a = _gpu_topk(s, 2048)
    b = _gpu_topk(s, 2048)
    assert np.array_equal(a, b)
    # documented order: an upper group in ascending index order, then the cut group,
    # in ascending index order or (pairwise cut) by score descending, index ascending;
    # every score of the upper group above every score of the cut group
    for bi in range(2):
        for ti in range(2):
            r = a[bi, ti]
            v = s[bi, ti][r]
            ok = False
            for p in range(len(r) + 1):
                if np.all(np.diff(r[:p]) > 0) and (np.all(np.diff(r[p:]) > 0) or _rank_ordered(r[p:], v[p:])) and (
                        p == 0 or p == len(r) or v[:p].min() > v[p:].max()):
                    ok = True
                    break
            assert ok, (bi, ti)


@pytest.mark.parametrize("T", [8192, 4096])          # the 1024- and the 256-thread kernel
def test_topk_cut_paths(T):
    """Rows built so that the bin holding the k-th largest score is taken whole, holds a
    few elements (ranked pairwise: at most 256 with 1024 threads, 64 with 256) or many
    (radix passes), or the row has no spread."""
    rng = np.random.default_rng(8)
    k = 1000
    rows = []
    base = rng.standard_normal(T).astype(np.float32)
    rows.append(base)                                          # a few elements in the cut bin
    r = np.arange(T, dtype=np.float32)                         # evenly spaced: every bin holds the same few
    rows.append(rng.permutation(r))
    crowd = base.copy()
    crowd[rng.choice(T, 3000, replace=False)] = 0.5            # ~3000 equal values straddle the cut
    rows.append(crowd)
    near = (1.0 + rng.integers(0, 200, T) * 2.0**-23).astype(np.float32)   # 200 adjacent floats
    near[0] = -1.0e6                                           # a wide range puts them all in one bin
    rows.append(near)
    rows.append(np.full(T, 7.0, np.float32))                   # no spread
    wide = base.copy()
    wide[5] = 3.0e38                                           # range beyond 1e30: single bin
    wide[6] = -3.0e38
    rows.append(wide)
    tiny = (base * 1e-33).astype(np.float32)                   # range below 1e-30
    rows.append(tiny)
    xk = np.sort(base)[-k]
    for m in (150, 400):                                       # m distinct values crowd the cut bin:
        crowded = base.copy()                                  # pairwise (150, 1024 threads) or radix
        pick = rng.choice(np.flatnonzero(base < xk), m, replace=False)
        crowded[pick] = (xk + np.arange(1, m + 1) * 2.0**-21 * abs(xk)).astype(np.float32)
        rows.append(crowded)
    s = np.stack(rows)[:, None, :]
    log(f"[topk] cut paths T={T}")
    for kk in (k, 1, 64, 65, 4096):
        _check_exact(s, kk, _gpu_topk(s, kk), None)
