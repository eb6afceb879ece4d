"""Key write and query preparation on the GPU, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def _gpu_quantize_rows(x_bf16: torch.Tensor):
    """Quantize [n, 128] rows through lk_quantize_keys into a fresh 1-sequence cache."""
    n = x_bf16.shape[0]
    cache = torch.full((1, n, 128), 0xAA, dtype=torch.uint8, device=DEV)
    scale = torch.full((1, n), -1.0, dtype=torch.float32, device=DEV)
    api.lk_quantize_keys(x_bf16.reshape(1, n, 128).to(DEV), cache, scale)
    torch.cuda.synchronize()
    return cache[0].cpu().numpy(), scale[0].cpu().numpy()


def _assert_same(bits: np.ndarray, what: str):
    x = _bits_to_bf16(bits)
    log(f"[quantize] {what}: {bits.shape[0]} rows")
    gc, gs = _gpu_quantize_rows(x)
    oc, os_ = O.quantize_rows(bits)
    bad = np.nonzero(np.any(gc != oc, axis=1) | (gs.view(np.uint32) != os_.view(np.uint32)))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first row {bad[0]}: gpu {gc[bad[0]][:8]} / {gs[bad[0]]} vs oracle {oc[bad[0]][:8]} / {os_[bad[0]]}"


def test_random_rows_bit_exact():
    g = torch.Generator().manual_seed(100)
    x = torch.randn(6000, 128, generator=g)
    x = x * torch.exp2(torch.randint(-20, 20, (6000, 1), generator=g).float())
    _assert_same(W.bf16_bits(x.to(torch.bfloat16)), "random rows, scales 2^-20..2^20")


def test_every_single_bf16_value_bit_exact():
    """Rows [v, 0, ..., 0] for every finite bf16 v with |v| < 2^120 (each rotates to +-v/sqrt(128))."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float()
    keep = (torch.isfinite(vals) & (vals.abs() < 2.0**120)).numpy()
    v = allbits[keep]
    rows = np.zeros((v.size, 128), np.uint16)
    rows[:, 0] = v
    rows[1::2, 77] = rows[1::2, 0]          # odd rows: the same value in a second slot
    rows[1::2, 0] = 0
    _assert_same(rows, "single-value rows over all finite bf16")


def test_pairs_exercise_rounding_bit_exact():
    """Rows [1, v, ...] and [v, -3, ...]: the rotation sums mix two magnitudes."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float()
    keep = (torch.isfinite(vals) & (vals != 0) & (vals.abs() <= 2.0**30) & (vals.abs() >= 2.0**-30)).numpy()
    v = allbits[keep][::3]
    rows = np.zeros((v.size, 128), np.uint16)
    one = W.bf16_bits(torch.tensor([1.0, -3.0, 0.5]).to(torch.bfloat16))
    rows[:, 0] = one[0]
    rows[:, 5] = v
    rows[::2, 64] = one[1]
    rows[1::2, 127] = one[2]
    _assert_same(rows, "two- and three-value rows")


def test_edge_rows_bit_exact():
    rows = []
    f = lambda a: W.bf16_bits(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    rows.append(f([0.0] * 128))                                   # zero row -> zeros, scale 2^-126
    rows.append(f([-0.0] * 128))
    rows.append(f([1.0] * 128))
    rows.append(f([(-1.0) ** i for i in range(128)]))
    rows.append(f([448.0 if i == 3 else 0.0 for i in range(128)]))
    rows.append(f([2.0**-100] * 64 + [-(2.0**-100)] * 64))
    rows.append(f([2.0**60 * (1 + i / 128) for i in range(128)]))
    rows.append(f([2.0**-30 if i % 2 else 2.0**8 for i in range(128)]))   # span 2^38
    rows.append(f([float(i - 64) for i in range(128)]))
    rows.append(f([1.0 + 2.0**-7] + [0.0] * 127))
    rows.append(f([2.0**-126, -(2.0**-133)] + [0.0] * 126))       # subnormal inputs
    _assert_same(np.stack(rows), "edge rows")


def test_positions_offsets_and_skipped_rows():
    g = torch.Generator().manual_seed(101)
    n_seq, n_rows, cap = 3, 5, 12
    x = torch.randn(n_seq, n_rows, 128, generator=g).to(torch.bfloat16)
    oc, os_ = O.quantize_rows(W.bf16_bits(x).reshape(-1, 128))
    oc = oc.reshape(n_seq, n_rows, 128)
    os_ = os_.reshape(n_seq, n_rows)
    # a cache with a larger sequence stride than its capacity (a slice of a wider buffer)
    big = torch.full((n_seq, cap + 4, 128), 0x5A, dtype=torch.uint8, device=DEV)
    bigs = torch.full((n_seq, cap + 4), 7.0, dtype=torch.float32, device=DEV)
    cache, scale = big[:, :cap], bigs[:, :cap]
    pos = torch.tensor([0, 9, -2], dtype=torch.int32)              # seq 1: rows 12,13 skipped; seq 2: rows -2,-1 skipped
    log("[quantize] positions with skipped rows")
    api.lk_quantize_keys(x.to(DEV), cache, scale, positions=pos.to(DEV))
    torch.cuda.synchronize()
    c, s = big.cpu().numpy(), bigs.cpu().numpy()
    for b in range(n_seq):
        for i in range(n_rows):
            p = int(pos[b]) + i
            if 0 <= p < cap:
                assert np.array_equal(c[b, p], oc[b, i]) and s[b, p] == os_[b, i], (b, i)
        written = {int(pos[b]) + i for i in range(n_rows)}
        for p in range(cap + 4):
            if p not in written or p >= cap:
                assert np.all(c[b, p] == 0x5A) and s[b, p] == 7.0, (b, p)
    # a fixed row offset
    log("[quantize] row_offset")
    api.lk_quantize_keys(x[:1].to(DEV), cache, scale, row_offset=4)
    torch.cuda.synchronize()
    assert np.array_equal(big[0, 4:9].cpu().numpy(), oc[0])


def test_queries_and_weight_fold_bit_exact():
    g = torch.Generator().manual_seed(102)
    n_tok = 37
    q = torch.randn(n_tok, 64, 128, generator=g).to(torch.bfloat16)
    w = torch.randn(n_tok, 64, generator=g) * 0.125
    log("[quantize] queries + fold")
    qs = torch.empty(n_tok, 64, device=DEV)
    q8, we = api.lk_quantize_queries(q.to(DEV), w.to(DEV), q_scale=qs)
    torch.cuda.synchronize()
    oc, os_ = O.quantize_rows(W.bf16_bits(q).reshape(-1, 128))
    ow = O.fold_weights(w.numpy().reshape(-1), os_)
    assert np.array_equal(q8.cpu().numpy().reshape(-1, 128), oc)
    assert np.array_equal(qs.cpu().numpy().reshape(-1).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(we.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32))


def test_prepare_equals_separate_calls():
    g = torch.Generator().manual_seed(103)
    x = torch.randn(3, 7, 128, generator=g).to(torch.bfloat16).to(DEV)
    q = torch.randn(5, 64, 128, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(5, 64, generator=g) * 0.125).to(DEV)
    pos = torch.tensor([0, 20, 41], dtype=torch.int32, device=DEV)
    c1 = torch.zeros(3, 48, 128, dtype=torch.uint8, device=DEV)
    s1 = torch.zeros(3, 48, device=DEV)
    c2, s2 = c1.clone(), s1.clone()
    log("[quantize] lk_prepare vs separate calls")
    api.lk_quantize_keys(x, c1, s1, positions=pos)
    q8a, wa = api.lk_quantize_queries(q, w)
    q8b, wb = api.lk_prepare(x, c2, s2, q, w, positions=pos)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(q8a, q8b) and torch.equal(wa.view(torch.int32), wb.view(torch.int32))
    # one job empty
    c3, s3 = torch.zeros_like(c1), torch.zeros_like(s1)
    api.lk_prepare(x[:, :0], c3, s3, q, w, positions=pos)
    q8c, wc = api.lk_prepare(x, c3, s3, q[:0], w[:0], positions=pos)
    torch.cuda.synchronize()
    assert torch.equal(c3, c1) and q8c.numel() == 0
