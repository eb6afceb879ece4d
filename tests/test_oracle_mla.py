"""Pins of the oracle's sparse MLA decode attention (reading R13) by closed forms:
one selected key returns its latent row, equal logits average the selected rows,
-1 slots and the order of the index list change nothing, a dominant logit selects
its row, two keys follow the logistic weight of their logit gap, and an empty list
returns zeros."""
import math

import numpy as np
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import workloads as W

H, DC, DR, T = 4, 512, 64, 40


def _bits(a):
    return W.bf16_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def _vals(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def _case(seed=0, qscale=1.0):
    rng = np.random.default_rng(seed)
    qc = _bits(rng.standard_normal((H, DC)) * qscale)
    qr = _bits(rng.standard_normal((H, DR)) * qscale)
    kv = _bits(rng.standard_normal((T, DC)))
    pe = _bits(rng.standard_normal((T, DR)))
    return qc, qr, kv, pe


def test_single_key_returns_its_row():
    qc, qr, kv, pe = _case(1)
    o = O.sparse_mla_row(qc, qr, kv, pe, np.array([7, -1, -1], np.int32), 0.1)
    assert np.array_equal(o, np.broadcast_to(_vals(kv[7]), (H, DC)))


def test_equal_logits_average_the_rows():
    qc, qr, kv, pe = _case(2)
    zq = np.zeros_like(qc)
    zr = np.zeros_like(qr)
    sel = np.array([3, 11, 29, 5], np.int32)
    o = O.sparse_mla_row(zq, zr, kv, pe, sel, 0.37)
    want = _vals(kv[sel]).mean(axis=0)
    assert np.allclose(o, np.broadcast_to(want, (H, DC)), rtol=0, atol=1e-14)


def test_unused_slots_and_order_do_not_matter():
    qc, qr, kv, pe = _case(3)
    a = O.sparse_mla_row(qc, qr, kv, pe, np.array([4, 9, 17, 33], np.int32), 0.05)
    b = O.sparse_mla_row(qc, qr, kv, pe, np.array([-1, 33, 9, -1, 4, 17, -1], np.int32), 0.05)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


def test_dominant_logit_selects_its_row():
    qc, qr, kv, pe = _case(4, qscale=0.0)
    # head 0 aligned with key 12's rotary part only: logit 1000 x scale for key 12, 0 for others
    qr = qr.copy()
    pe = pe.copy()
    pe[:] = _bits(np.zeros((T, DR)))
    pe[12, 0] = _bits([1.0])[0]
    qr[0, 0] = _bits([1000.0])[0]
    o = O.sparse_mla_row(qc, qr, kv, pe, np.array([2, 12, 30], np.int32), 1.0)
    assert np.allclose(o[0], _vals(kv[12]), rtol=0, atol=1e-300 + 1e-12)
    # the other heads see equal logits: the average of the three rows
    assert np.allclose(o[1], _vals(kv[[2, 12, 30]]).mean(axis=0), atol=1e-14)


def test_two_keys_follow_the_logistic_weight():
    qc, qr, kv, pe = _case(5, qscale=0.0)
    pe = pe.copy()
    qr = qr.copy()
    pe[:] = _bits(np.zeros((T, DR)))
    pe[1, 5] = _bits([2.0])[0]
    qr[:, 5] = _bits([0.75] * H)
    scale = 0.5          # logit gap: 0.5 * 0.75 * 2 = 0.75 in favour of key 1
    o = O.sparse_mla_row(qc, qr, kv, pe, np.array([1, 6], np.int32), scale)
    p1 = 1.0 / (1.0 + math.exp(-0.75))
    want = p1 * _vals(kv[1]) + (1 - p1) * _vals(kv[6])
    assert np.allclose(o, np.broadcast_to(want, (H, DC)), rtol=1e-13, atol=1e-13)


def test_empty_list_returns_zeros():
    qc, qr, kv, pe = _case(6)
    o = O.sparse_mla_row(qc, qr, kv, pe, np.array([-1, -1], np.int32), 0.1)
    assert np.all(o == 0)
