"""Pins for the CPU oracle: each test checks it against something other than itself
(a library routine, a closed form, exact rational arithmetic, a hand-worked case or
an invariant the pages state).  CPU only."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import oracle as O


def _hex_codes(spec: str):
    out = []
    for tok in spec.split():
        if "*" in tok:
            h, n = tok.split("*")
            out += [int(h, 16)] * int(n)
        else:
            out.append(int(tok, 16))
    return out


def _bf16_bits_of(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(values, dtype=torch.float32)), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- fp8 codec
def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert math.isnan(got[c]) and math.isnan(ref[c])
        else:
            assert got[c] == ref[c] and math.copysign(1, got[c]) == math.copysign(1, ref[c]), hex(c)


def test_e4m3_roundtrip_every_finite_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert O.e4m3_encode(O.e4m3_decode(np.uint8(c))[()]) == c


def test_e4m3_encode_matches_torch_on_all_bf16_values_and_midpoints():
    # every finite bf16 value with |v| <= 448, plus every midpoint between adjacent codes
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    keep = torch.isfinite(vals) & (vals.abs() <= 448)
    vals = vals[keep]
    pos = np.array([O.e4m3_decode(np.uint8(c))[()] for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    mids = torch.tensor(np.concatenate([mids, -mids]), dtype=torch.float32)
    allv = torch.cat([vals, mids])
    ref = allv.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    lib_enc = [O.e4m3_encode(float(v)) for v in allv.tolist()]
    mism = [(float(allv[i]), ref[i], lib_enc[i]) for i in range(len(ref)) if ref[i] != lib_enc[i]]
    assert not mism, mism[:10]
    assert len(allv) > 34000


def test_e4m3_encoder_edges(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e4m3_encoder_edges.json")))
    for c in g["cases"]:
        assert O.e4m3_encode(c["v"]) == int(c["code"], 16), c


# ---------------------------------------------------------------- bf16 rounding
def _bf16_nearest_bruteforce(p: float) -> int:
    """Nearest bf16 by exact comparison with the two neighbouring bit patterns."""
    f32 = struct.unpack("<I", struct.pack("<f", np.float32(p)))[0]
    hi16 = f32 >> 16
    cands = {(hi16 + d) & 0xFFFF for d in (-1, 0, 1, 2)}
    best = None
    for c in sorted(cands):
        v = O.bf16_decode(c)
        if not math.isfinite(v):
            continue
        if math.copysign(1, v) != math.copysign(1, p) and v != 0:
            continue
        dist = abs(Fraction(v) - Fraction(p))
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_round_single_rounding_hand_case():
    # 1 + 2^-8 + 2^-30 is above the midpoint 1 + 2^-8: nearest bf16 is 1 + 2^-7 (0x3F81).
    # A detour through binary32 would first round to 1 + 2^-8 and then tie to 1.0.
    assert O.bf16_round(1.0 + 2.0**-8 + 2.0**-30) == 0x3F81
    assert O.bf16_round(1.0 + 2.0**-8) == 0x3F80      # exact tie -> even
    assert O.bf16_round(1.0 + 3 * 2.0**-8) == 0x3F82  # exact tie -> even (up)


def test_bf16_round_matches_torch_for_binary32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_matches_bruteforce_on_doubles():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(400) * np.exp2(rng.integers(-20, 20, 400))
    for v in x:
        assert O.bf16_round(float(v)) == _bf16_nearest_bruteforce(float(v)), v


# ---------------------------------------------------------------- Hadamard rotation
def test_hadamard_is_sylvester_matrix():
    H = np.array([[O.hadamard_entry(j, i) for i in range(128)] for j in range(128)])
    assert np.array_equal(H, scipy.linalg.hadamard(128))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, 128 * np.eye(128, dtype=H.dtype))


def test_rotation_scale_is_correctly_rounded():
    C = O.rotation_scale(128)
    assert struct.unpack("<Q", struct.pack("<d", C))[0] == 0x3FB6A09E667F3BCD
    half_ulp = Fraction(math.ulp(C)) / 2
    lo, hi = Fraction(C) - half_ulp, Fraction(C) + half_ulp
    assert lo * lo < Fraction(1, 128) < hi * hi        # 2^-3.5 lies within half an ulp
    assert O.rotation_scale(1) == 1.0


def test_rotation_is_exact_sum_times_scale():
    """p_j equals fl64(exact(sum_i H[j][i] x_i) * C64), by exact rational arithmetic."""
    rng = np.random.default_rng(3)
    C = Fraction(O.rotation_scale(128))
    H = scipy.linalg.hadamard(128)
    for _ in range(3):
        xb = torch.randn(128, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(torch.bfloat16)
        bits = xb.view(torch.int16).numpy().view(np.uint16)
        xs = [Fraction(float(v)) for v in xb.float().tolist()]
        p = O.rotate_row(bits)
        for j in range(128):
            r = sum(int(H[j, i]) * xs[i] for i in range(128))
            assert p[j] == float(r * C), j


def test_rotation_preserves_dot_products():
    """Page 'Hadamard rotation': the transform is orthonormal, so q.k is unchanged."""
    g = torch.Generator().manual_seed(4)
    for _ in range(20):
        a = torch.randn(128, generator=g).to(torch.bfloat16)
        b = torch.randn(128, generator=g).to(torch.bfloat16)
        pa = O.rotate_row(a.view(torch.int16).numpy().view(np.uint16))
        pb = O.rotate_row(b.view(torch.int16).numpy().view(np.uint16))
        ref = float(torch.dot(a.double(), b.double()))
        assert abs(float(np.dot(pa, pb)) - ref) <= 1e-12 * (np.linalg.norm(pa) * np.linalg.norm(pb))
        assert abs(np.linalg.norm(pa) - float(a.double().norm())) <= 1e-12 * float(a.double().norm())


def test_rotation_rejects_rows_beyond_exact_range():
    bits = _bf16_bits_of([1.0] + [0.0] * 126 + [2.0**-40])
    with pytest.raises(O.OracleRangeError):
        O.rotate_row(bits)


# ---------------------------------------------------------------- quantizer
def test_quantize_worked_examples(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "quantize_worked_examples.json")))
    for c in g["cases"]:
        d = c["d"]
        if c["x"] == "e0":
            x = [1.0] + [0.0] * (d - 1)
        elif c["x"] == "ones":
            x = [1.0] * d
        else:
            x = c["x"]
        codes, scales = O.quantize_rows(_bf16_bits_of(x).reshape(1, d))
        assert list(codes[0]) == _hex_codes(c["codes"]), c
        assert scales[0] == 2.0 ** c["scale_exp"], c


def test_scale_exponent_closed_form_all_bf16():
    """j* = max(-126, e - 8 + [m > 96]) for normal A = (1 + m/128) 2^e; -126 for subnormal A."""
    for bits in range(0x0001, 0x7F80):
        A = O.bf16_decode(bits)
        E = bits >> 7
        m = bits & 0x7F
        want = -126 if E == 0 else max(-126, (E - 127) - 8 + (1 if m > 96 else 0))
        assert O.scale_exponent(A) == want, hex(bits)
    assert O.scale_exponent(0.0) == -126


def test_quantize_scale_equivariance():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(8, 128, generator=g).to(torch.bfloat16)
    c0, s0 = O.quantize_rows(x.view(torch.int16).numpy().view(np.uint16))
    for m in (-7, -1, 1, 3, 9):
        xm = (x.float() * 2.0**m).to(torch.bfloat16)
        assert torch.equal(xm.float(), x.float() * 2.0**m)
        cm, sm = O.quantize_rows(xm.view(torch.int16).numpy().view(np.uint16))
        assert np.array_equal(cm, c0) and np.array_equal(sm, s0 * np.float32(2.0**m))


def test_quantize_exact_zero_sums_are_plus_zero():
    """Closed form of the row [-0, +0, 1, 1, 0, ...]: r_j = s(j & 2) + s(j & 3) with
    s(m) = (-1)^popcount(m), so every odd j sums to exactly zero (code 0x00, never 0x80)
    and every even j to +-2 (2 / sqrt(128) -> bf16 0.1767578125 = 362 * 2^-11, so
    scale 2^-11 and code 0x7B (352) or 0xFB).  The same with -0 in every empty slot."""
    exp = np.array([0 if j & 1 else (0xFB if j & 2 else 0x7B) for j in range(128)], np.uint8)
    one = np.uint16(0x3F80)
    for fill in (0x0000, 0x8000):
        row = np.full(128, fill, np.uint16)
        row[0], row[1], row[2], row[3] = 0x8000, 0x0000, one, one
        codes, scales = O.quantize_rows(row[None, :])
        assert np.array_equal(codes[0], exp)
        assert scales[0] == np.float32(2.0 ** -11)


def test_quantize_properties_random_rows():
    g = torch.Generator().manual_seed(6)
    x = torch.randn(256, 128, generator=g).to(torch.bfloat16)
    codes, scales = O.quantize_rows(x.view(torch.int16).numpy().view(np.uint16))
    sb = scales.view(np.uint32)
    assert np.all((sb & 0x7FFFFF) == 0)                      # e8m0: power of two
    assert not np.any((codes & 0x7F) == 0x7F)                # never NaN
    dec = O.e4m3_decode(codes)
    mx = np.abs(dec).max(axis=1)
    assert np.all(mx >= 224) and np.all(mx <= 448)           # amax lands in (224, 448] before rounding
    # dequantized rows approximate the rotated rows (fp8 relative error <= 2^-4 of amax)
    for r in range(8):
        p = O.rotate_row(x[r].view(torch.int16).numpy().view(np.uint16))
        deq = dec[r] * scales[r]
        assert np.max(np.abs(deq - p)) <= 2.0**-4 * np.max(np.abs(p)) + 1e-30


# ---------------------------------------------------------------- weight fold
def test_fold_weights_constant_and_power_of_two_scales():
    c32 = struct.unpack("<f", struct.pack("<I", 0x3DB504F3))[0]
    w = np.array([1.0, -1.0, 0.125, 3.0], dtype=np.float32)
    qs = np.array([2.0**-8, 2.0**-7, 1.0, 2.0**-10], dtype=np.float32)
    out = O.fold_weights(w, qs)
    assert out[0] == np.float32(c32 * 2.0**-8)
    assert out[1] == np.float32(-c32 * 2.0**-7)
    assert out[2] == np.float32(c32 / 8)
    # 3 * c32 rounds once in binary32; scaling by a power of two is exact
    assert out[3] == np.float32(np.float32(3.0) * np.float32(c32)) * np.float32(2.0**-10)


# ---------------------------------------------------------------- score
def test_score_hand_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "score_hand_cases.json")))
    for c in g["cases"]:
        H, d = c["H"], c["d"]
        q8 = np.array([int(h, 16) for h in c["q8"]], dtype=np.uint8).reshape(H, d)
        k8 = np.array([int(h, 16) for h in c["k8"]], dtype=np.uint8).reshape(-1, d)
        ks = np.array(c["k_scale"], dtype=np.float32)
        w = np.array(c["w_eff"], dtype=np.float32)
        T = k8.shape[0]
        s = O.score_row(q8, w, k8, ks, T, T)
        want = np.array(c["scores"])
        assert np.array_equal(s, want), (c["name"], s)
        top = O.topk(s, T, c["k"])
        assert sorted(top.tolist()) == sorted(c["topk"]), c["name"]


def _random_quantized(seed, H=8, T=40):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(T, 128, generator=g).to(torch.bfloat16)
    q8, qs = O.quantize_rows(q.view(torch.int16).numpy().view(np.uint16))
    k8, ks = O.quantize_rows(k.view(torch.int16).numpy().view(np.uint16))
    w = (torch.randn(H, generator=g) * 0.125).numpy()
    return q8, qs, k8, ks, w.astype(np.float32)


def test_score_nonnegative_when_weights_nonnegative():
    q8, qs, k8, ks, w = _random_quantized(7)
    s = O.score_row(q8, np.abs(O.fold_weights(w, qs)), k8, ks, len(ks), len(ks))
    assert np.all(s >= 0)


def test_score_key_scale_power_of_two_is_exact():
    q8, qs, k8, ks, w = _random_quantized(8)
    we = O.fold_weights(w, qs)
    s0 = O.score_row(q8, we, k8, ks, len(ks), len(ks))
    ks2 = ks.copy()
    ks2[::3] *= np.float32(2.0**5)
    s1 = O.score_row(q8, we, k8, ks2, len(ks), len(ks))
    assert np.array_equal(s1[::3], s0[::3] * 2.0**5)
    mask = np.ones(len(ks), bool)
    mask[::3] = False
    assert np.array_equal(s1[mask], s0[mask])


def test_score_key_permutation_equivariance():
    q8, qs, k8, ks, w = _random_quantized(9)
    we = O.fold_weights(w, qs)
    perm = np.random.default_rng(0).permutation(len(ks))
    s0 = O.score_row(q8, we, k8, ks, len(ks), len(ks))
    s1 = O.score_row(q8, we, k8[perm], ks[perm], len(ks), len(ks))
    assert np.array_equal(s1, s0[perm])
    t0 = O.topk(s0, len(ks), 5)
    t1 = O.topk(s1, len(ks), 5)
    assert sorted(perm[t1].tolist()) == sorted(t0.tolist())


def test_score_linear_in_weights():
    q8, qs, k8, ks, w = _random_quantized(10)
    w1 = np.float32(np.arange(8) - 3.5) * np.float32(2.0**-12)
    w2 = np.float32(np.arange(8) % 3) * np.float32(2.0**-11)
    T = len(ks)
    s12 = O.score_row(q8, (w1 + w2).astype(np.float32), k8, ks, T, T)
    s1 = O.score_row(q8, w1, k8, ks, T, T)
    s2 = O.score_row(q8, w2, k8, ks, T, T)
    assert np.allclose(s12, s1 + s2, rtol=1e-13, atol=1e-13 * np.abs(s12).max())


def test_score_one_hot_head_is_relu_matmul():
    """With w = e_h the score reduces to k_scale * w_h * ReLU(Q_h K^T), a plain matmul."""
    q8, qs, k8, ks, w = _random_quantized(11)
    Qd = torch.from_numpy(O.e4m3_decode(q8))
    Kd = torch.from_numpy(O.e4m3_decode(k8))
    for h in (0, 5):
        we = np.zeros(8, np.float32)
        we[h] = np.float32(0.75)
        s = O.score_row(q8, we, k8, ks, len(ks), len(ks))
        ref = torch.relu(torch.matmul(Kd, Qd[h])) * 0.75 * torch.from_numpy(ks.astype(np.float64))
        assert np.array_equal(s, ref.numpy())


def test_score_mask_prefix_is_minus_inf():
    q8, qs, k8, ks, w = _random_quantized(12)
    we = O.fold_weights(w, qs)
    s = O.score_row(q8, we, k8, ks, 40, 17)
    assert np.all(np.isneginf(s[17:])) and np.all(np.isfinite(s[:17]))
    assert np.all(s[17:].view(np.uint64) == 0xFFF0000000000000)


def test_valid_len_rules():
    assert O.valid_len(16384, -1, False, 16383, 0) == 16384          # plain decode: no mask
    assert O.valid_len(16384, 5000, False, 4999, 0) == 5000          # ragged
    assert O.valid_len(16384, 20000, False, 0, 0) == 16384           # lengths clamp to T
    assert O.valid_len(4096, -1, True, 0, 0) == 1                    # causal first row
    assert O.valid_len(4096, -1, True, 0, 4095) == 4096
    assert O.valid_len(16384, -1, True, 12288, 5) == 12294           # chunked prefill
    assert O.valid_len(100, -1, True, -5, 0) == 0


# ---------------------------------------------------------------- top-k
def test_topk_matches_torch_values():
    rng = np.random.default_rng(13)
    for L, k in ((1000, 256), (5000, 2048), (16384, 2048)):
        v = rng.standard_normal(L).astype(np.float32)
        idx = O.topk(v, L, k)
        ref = torch.topk(torch.from_numpy(v), k).values.numpy()
        assert np.array_equal(np.sort(v[idx]), np.sort(ref))
        assert len(set(idx.tolist())) == k


def test_topk_ties_go_to_lower_index_bruteforce():
    rng = np.random.default_rng(14)
    for _ in range(50):
        L = int(rng.integers(1, 30))
        v = rng.integers(-3, 3, L).astype(np.float32)
        k = int(rng.integers(1, 12))
        want = [i for _, i in sorted((-float(v[i]), i) for i in range(L))][:k]
        got = O.topk(v, L, k)
        assert sorted(got[got >= 0].tolist()) == sorted(want)
        assert np.all(got[min(k, L):] == -1)


def test_topk_signed_zero_and_short_rows():
    v = np.array([-0.0, 0.0, -1.0], dtype=np.float32)
    assert O.topk(v, 3, 1).tolist() == [0]
    assert sorted(O.topk(v, 3, 5).tolist()) == [-1, -1, 0, 1, 2]
    assert O.topk(v, 0, 2).tolist() == [-1, -1]
    assert sorted(O.topk(np.arange(10, dtype=np.float32), 7, 3).tolist()) == [4, 5, 6]
