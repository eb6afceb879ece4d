"""Pins of the oracle's RoPE (reading R12: pairs (i, i + 32) of the leading 64
features, fp32 products and sum, one rounding to bf16), independent of its own code:
exact special angles, a hand-computed value, the non-interleaved pairing, agreement
with an exact complex product to one bf16 ulp, untouched trailing features, and the
norm of each rotated pair."""
import numpy as np
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import workloads as W


def _bf16(vals) -> np.ndarray:
    return W.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def _val(bits) -> np.ndarray:
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).float().numpy()


def _rand_row(rng, zeros=False):
    v = rng.standard_normal(128).astype(np.float32) * np.exp2(rng.integers(-8, 8, 128)).astype(np.float32)
    if not zeros:
        v[v == 0] = 1.0
    return _bf16(v)


def test_identity_angle_leaves_the_row_unchanged():
    rng = np.random.default_rng(20)
    for _ in range(20):
        x = _rand_row(rng)
        y = O.rope_row(x, np.ones(32, np.float32), np.zeros(32, np.float32))
        assert np.array_equal(y, x)


def test_quarter_turn_swaps_and_negates_exactly():
    rng = np.random.default_rng(21)
    for _ in range(20):
        x = _rand_row(rng)
        y = O.rope_row(x, np.zeros(32, np.float32), np.ones(32, np.float32))
        xv, yv = _val(x), _val(y)
        assert np.array_equal(yv[:32], -xv[32:64])
        assert np.array_equal(yv[32:64], xv[:32])
        assert np.array_equal(y[64:], x[64:])


def test_hand_computed_pair():
    # x0 = 1.5, x32 = -2, cos = 0.5, sin = 0.25:
    #   y0  = 1.5 * 0.5 - (-2) * 0.25 = 0.75 + 0.5 = 1.25
    #   y32 = 1.5 * 0.25 + (-2) * 0.5 = 0.375 - 1 = -0.625
    x = np.zeros(128, np.uint16)
    x[0], x[32] = _bf16([1.5, -2.0])
    c = np.zeros(32, np.float32)
    s = np.zeros(32, np.float32)
    c[0], s[0] = 0.5, 0.25
    c[1:] = 1.0
    y = _val(O.rope_row(x, c, s))
    assert y[0] == 1.25 and y[32] == -0.625
    assert np.all(y[1:32] == 0) and np.all(y[33:] == 0)


def test_pairs_are_not_interleaved():
    # one unit at feature 0 turned by 90 degrees lands on feature 32 (half split), not
    # on feature 1 (interleaved pairs)
    x = np.zeros(128, np.uint16)
    x[0] = _bf16([1.0])[0]
    y = _val(O.rope_row(x, np.zeros(32, np.float32), np.ones(32, np.float32)))
    assert y[32] == 1.0 and y[1] == 0.0 and y[0] == 0.0


def test_within_one_ulp_of_the_exact_complex_product():
    rng = np.random.default_rng(22)
    for _ in range(50):
        x = _rand_row(rng)
        ang = rng.uniform(-np.pi, np.pi, 32)
        c = np.cos(ang).astype(np.float32)
        s = np.sin(ang).astype(np.float32)
        y = _val(O.rope_row(x, c, s)).astype(np.float64)
        xv = _val(x).astype(np.float64)
        z = (xv[:32] + 1j * xv[32:64]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
        exact = np.concatenate([z.real, z.imag])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
        # fp32 products and sum can cancel: allow the fp32 error of the two products too
        slack = 2.0 ** -23 * (np.abs(np.concatenate([xv[:32] * c, xv[:32] * s])) +
                              np.abs(np.concatenate([xv[32:64] * s, xv[32:64] * c])))
        assert np.all(np.abs(y[:64] - exact) <= ulp + slack)
        assert np.array_equal(y[64:], xv[64:])


def test_rotated_pairs_keep_their_norm():
    rng = np.random.default_rng(23)
    x = _rand_row(rng)
    ang = rng.uniform(-np.pi, np.pi, 32)
    y = _val(O.rope_row(x, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))).astype(np.float64)
    xv = _val(x).astype(np.float64)
    n0 = np.hypot(xv[:32], xv[32:64])
    n1 = np.hypot(y[:32], y[32:64])
    assert np.all(np.abs(n1 - n0) <= 2.0 ** -6 * n0 + 1e-30)


def test_batch_rows_pick_their_table_row():
    rng = np.random.default_rng(24)
    x = np.stack([_rand_row(rng) for _ in range(6)])
    ang = rng.uniform(-np.pi, np.pi, (3, 32))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    codes, scales = O.rope_quantize_rows(x, c, s, rows_per_table_row=2)
    for r in range(6):
        y = O.rope_row(x[r], c[r // 2], s[r // 2])
        c1, s1 = O.quantize_rows(y[None])
        assert np.array_equal(codes[r], c1[0]) and scales[r] == s1[0]
