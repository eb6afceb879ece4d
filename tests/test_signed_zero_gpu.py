"""Signed zeros through every quantizing entry point, bit-exact against the oracle.

A Hadamard sum that is exactly zero is +0 by definition (page "Hadamard rotation": the
rotated feature is a plain sum), so its e4m3fn code is 0x00 whatever signs the zero
inputs carried; only a nonzero value that rounds to zero keeps its sign (0x80).  Rows
here mix -0 and +0 inputs with nonzero features whose sums cancel exactly, and RoPE
tables with negative cosines turn zero feature pairs into -0 before the rotation.
The entry points covered: lk_quantize_keys, lk_quantize_queries, lk_prepare with and
without RoPE, and the query and new key inside lk_decode_score with and without RoPE.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

NEG0 = 0x8000


def _bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def _f(vals) -> np.ndarray:
    return W.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def zero_rich_rows(seed: int, n: int) -> np.ndarray:
    """n rows of bf16 bits in which exact cancellation and signed zeros are common."""
    rng = np.random.default_rng(seed)
    rows = []
    # the fixed cases first
    r = np.zeros(128, np.uint16); r[0] = NEG0; r[2:4] = _f([1.0, 1.0]); rows.append(r)
    r = np.full(128, NEG0, np.uint16); r[127] = _f([1.0])[0]; rows.append(r)
    r = np.full(128, NEG0, np.uint16); r[5] = _f([-2.0])[0]; r[77] = _f([2.0])[0]; rows.append(r)
    r = np.zeros(128, np.uint16); r[::2] = NEG0; r[64:66] = _f([3.0, -3.0]); rows.append(r)
    r = np.full(128, NEG0, np.uint16); r[:8] = _f([1, 1, 1, 1, -1, -1, -1, -1]); rows.append(r)
    while len(rows) < n:
        kind = len(rows) % 3
        if kind == 0:      # small integers, half of them zeros of random sign
            v = rng.choice([1.0, -1.0, 2.0, -2.0, 0.5, -0.5, 3.0, -3.0], 128)
            bits = _f(v)
            z = rng.random(128) < 0.5
            bits[z] = np.where(rng.random(z.sum()) < 0.5, NEG0, 0).astype(np.uint16)
        elif kind == 1:    # Gaussian values with 30% signed zeros
            bits = _f(rng.standard_normal(128) * 2.0 ** rng.integers(-8, 8))
            z = rng.random(128) < 0.3
            bits[z] = np.where(rng.random(z.sum()) < 0.5, NEG0, 0).astype(np.uint16)
        else:              # values copied to xor-partners, negated or not, among zeros
            bits = np.where(rng.random(128) < 0.5, NEG0, 0).astype(np.uint16)
            m = int(rng.integers(1, 128))
            for i in rng.choice(128, 6, replace=False):
                v = _f([float(rng.choice([1.0, 1.5, 0.75, 6.0]))])[0]
                bits[i] = v
                bits[i ^ m] = v ^ (NEG0 if rng.random() < 0.5 else 0)
        rows.append(bits.astype(np.uint16))
    return np.stack(rows[:n])


def negative_cos_tables(seed: int, n: int):
    """cos < 0 on every entry (angles in (pi/2, pi)), so a zero pair rotates to -0."""
    rng = np.random.default_rng(seed)
    ang = rng.uniform(0.55 * np.pi, 0.95 * np.pi, (n, 32))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _with_zero_pairs(rows: np.ndarray, seed: int) -> np.ndarray:
    """Zero both features of some RoPE pairs (i, i + 32), i < 32, with random zero signs."""
    rng = np.random.default_rng(seed)
    out = rows.copy()
    for r in out:
        for i in rng.choice(32, 10, replace=False):
            r[i] = NEG0 if rng.random() < 0.5 else 0
            r[i + 32] = NEG0 if rng.random() < 0.5 else 0
    return out


def _same(got_codes, got_scales, ref_codes, ref_scales, what):
    got_codes = np.asarray(got_codes).reshape(ref_codes.shape)
    bad = np.nonzero(np.any(got_codes != ref_codes, axis=1) |
                     (np.asarray(got_scales).reshape(-1).view(np.uint32) != ref_scales.view(np.uint32)))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows differ; first {bad[0]}: gpu {got_codes[bad[0]][:16]} "
                           f"oracle {ref_codes[bad[0]][:16]}")


def test_quantize_keys_and_queries():
    rows = zero_rich_rows(1, 64 * 6)
    oc, os_ = O.quantize_rows(rows)
    n = rows.shape[0]
    log(f"[signed zero] lk_quantize_keys, {n} rows")
    cache = torch.full((1, n, 128), 0xAA, dtype=torch.uint8, device=DEV)
    scale = torch.full((1, n), -1.0, dtype=torch.float32, device=DEV)
    api.lk_quantize_keys(_bits_to_bf16(rows).reshape(1, n, 128).to(DEV), cache, scale)
    torch.cuda.synchronize()
    _same(cache[0].cpu().numpy(), scale[0].cpu().numpy(), oc, os_, "lk_quantize_keys")

    log("[signed zero] lk_quantize_queries")
    q = _bits_to_bf16(rows).reshape(6, 64, 128)
    w = torch.randn(6, 64, generator=torch.Generator().manual_seed(7)) * 0.125
    qs = torch.empty(6, 64, device=DEV)
    q8, we = api.lk_quantize_queries(q.to(DEV), w.to(DEV), q_scale=qs)
    torch.cuda.synchronize()
    _same(q8.cpu().numpy(), qs.cpu().numpy(), oc, os_, "lk_quantize_queries")
    ow = O.fold_weights(w.numpy().reshape(-1), os_)
    assert np.array_equal(we.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32))


@pytest.mark.parametrize("rope", [False, True])
def test_prepare(rope):
    n_seq, n_rows, n_tok = 2, 96, 3
    krows = _with_zero_pairs(zero_rich_rows(2, n_seq * n_rows), 3)
    qrows = _with_zero_pairs(zero_rich_rows(4, n_tok * 64), 5)
    w = torch.randn(n_tok, 64, generator=torch.Generator().manual_seed(8)) * 0.125
    cache = torch.zeros(n_seq, n_rows + 4, 128, dtype=torch.uint8, device=DEV)
    cscale = torch.zeros(n_seq, n_rows + 4, device=DEV)
    qscale = torch.empty(n_tok, 64, device=DEV)
    kr = qr = None
    if rope:
        kc, ks = negative_cos_tables(6, n_seq * n_rows)
        qc, qsn = negative_cos_tables(7, n_tok)
        kr = (torch.from_numpy(kc).to(DEV), torch.from_numpy(ks).to(DEV))
        qr = (torch.from_numpy(qc).to(DEV), torch.from_numpy(qsn).to(DEV))
        ok, oks = O.rope_quantize_rows(krows, kc, ks)
        oq, oqs = O.rope_quantize_rows(qrows, qc, qsn, rows_per_table_row=64)
        # the RoPE step itself produces -0 inputs to the rotation here
        assert any(np.any(O.rope_row(r, kc[i], ks[i]) == NEG0) for i, r in enumerate(krows[:8]))
    else:
        ok, oks = O.quantize_rows(krows)
        oq, oqs = O.quantize_rows(qrows)
    log(f"[signed zero] lk_prepare rope={rope}")
    q8, we = api.lk_prepare(_bits_to_bf16(krows).reshape(n_seq, n_rows, 128).to(DEV), cache, cscale,
                            _bits_to_bf16(qrows).reshape(n_tok, 64, 128).to(DEV), w.to(DEV), row_offset=2,
                            q_scale=qscale, k_rope=kr, q_rope=qr)
    torch.cuda.synchronize()
    _same(cache[:, 2:2 + n_rows].cpu().numpy().reshape(-1, 128),
          cscale[:, 2:2 + n_rows].cpu().numpy(), ok, oks, "lk_prepare keys")
    _same(q8.cpu().numpy().reshape(-1, 128), qscale.cpu().numpy(), oq, oqs, "lk_prepare queries")
    ow = O.fold_weights(w.numpy().reshape(-1), oqs)
    assert np.array_equal(we.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32))


@pytest.mark.parametrize("rope", [False, True])
def test_decode_score_query_and_new_key(rope):
    """The fused decode step quantizes its query (64 heads per row) and its new key
    (written at slot L - 1) itself; both must carry the oracle's bytes."""
    B, T = 6, 1100                                # two key blocks per row: new key in the second
    qrows = _with_zero_pairs(zero_rich_rows(9, B * 64), 10)
    krows = _with_zero_pairs(zero_rich_rows(11, B), 12)
    w = torch.randn(B, 64, generator=torch.Generator().manual_seed(13)) * 0.125
    g = torch.Generator().manual_seed(14)
    prefix = torch.randn(B, T, 128, generator=g).to(torch.bfloat16)
    cache = torch.zeros(B, T, 128, dtype=torch.uint8, device=DEV)
    cscale = torch.zeros(B, T, device=DEV)
    api.lk_quantize_keys(prefix.to(DEV), cache, cscale)
    lens = torch.tensor([1, 2, 1024, 1025, 1099, 1100], dtype=torch.int32)
    q8 = torch.empty(B, 64, 128, dtype=torch.uint8, device=DEV)
    we = torch.empty(B, 64, device=DEV)
    rr = None
    if rope:
        c, s = negative_cos_tables(15, B)
        rr = (torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV))
        oq, oqs = O.rope_quantize_rows(qrows, c, s, rows_per_table_row=64)
        ok, oks = O.rope_quantize_rows(krows, c, s)
    else:
        oq, oqs = O.quantize_rows(qrows)
        ok, oks = O.quantize_rows(krows)
    log(f"[signed zero] lk_decode_score rope={rope}")
    api.lk_decode_score(_bits_to_bf16(qrows).reshape(B, 64, 128).to(DEV), w.to(DEV),
                        _bits_to_bf16(krows).reshape(B, 128).to(DEV), cache, cscale, T,
                        seq_len=lens.to(DEV), q_fp8_out=q8, w_eff_out=we, rope=rr)
    torch.cuda.synchronize()
    got = q8.cpu().numpy().reshape(-1, 128)
    bad = np.nonzero(np.any(got != oq, axis=1))[0]
    assert bad.size == 0, f"query codes: {bad.size} rows differ, first {bad[0]}"
    ow = O.fold_weights(w.numpy().reshape(-1), oqs)
    assert np.array_equal(we.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32)), "folded weights"
    c = cache.cpu().numpy()
    s = cscale.cpu().numpy()
    for b in range(B):
        L = int(lens[b])
        assert np.array_equal(c[b, L - 1], ok[b]), f"new key bytes, row {b} (slot {L - 1})"
        assert s[b, L - 1] == oks[b], f"new key scale, row {b}"
