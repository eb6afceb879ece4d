"""The measurement probes on the GPU.

* lk_probe_read touches every word of its buffer exactly once (the XOR of what it
  writes equals the XOR of the buffer).
* lk_probe_fp8_mfma_score: on small dyadic values, where every partial sum is exact in
  any accumulator, it equals the oracle's scores (this pins its operand layout); on
  the quantized decode workload it reports how far the fp8 matrix core's accumulation
  lands from the exact scores, next to the f16 path the library uses (which must stay
  within the 1e-5 bound).  This is the measurement behind the choice of f16 MFMA for
  the contraction.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import _lib, api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, gpu_pipeline, log, tol

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _probe_scores(q8, w_eff, cache, cache_scale, T, seq_len=None):
    lib = _lib.load()
    B = q8.shape[0]
    scores = torch.empty((B, T), dtype=torch.float32, device=DEV)
    rows = _lib.LkRows(B, 1, T, 0, seq_len.data_ptr() if seq_len is not None else None, 0)
    st = lib.lk_probe_fp8_mfma_score(q8.data_ptr(), w_eff.data_ptr(), cache.data_ptr(), cache_scale.data_ptr(),
                                     cache.stride(0) // 128, ctypes.byref(rows), scores.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    _lib.check("lk_probe_fp8_mfma_score", st)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def test_read_probe_covers_the_buffer_once():
    g = torch.Generator(device=DEV).manual_seed(3)
    n = (3 << 20) + 48                                  # not a multiple of the block span
    buf = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=DEV, generator=g)
    blocks = 37
    sink = torch.zeros(blocks * 4, dtype=torch.int32, device=DEV)
    log("[probe] read")
    st = _lib.load().lk_probe_read(buf.data_ptr(), n, sink.data_ptr(), blocks, torch.cuda.current_stream().cuda_stream)
    _lib.check("lk_probe_read", st)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_fp8_probe_layout_on_exact_values():
    """Codes of {0, +-0.5, +-1, +-2} and power-of-two weights and key scales: every
    product and partial sum is a small dyadic number, exact whatever the accumulator,
    so the probe must reproduce the oracle to float32 rounding of the head sum."""
    rng = np.random.default_rng(11)
    vals = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)
    B, T = 3, 300
    q8 = rng.choice(vals, (B, 64, 128))
    k8 = rng.choice(vals, (B, T, 128))
    w = np.ldexp(1.0, rng.integers(-6, 0, (B, 64))).astype(np.float32) * rng.choice([-1.0, 1.0], (B, 64)).astype(np.float32)
    ks = np.ldexp(1.0, rng.integers(-3, 3, (B, T))).astype(np.float32)
    log("[probe] fp8 MFMA layout on exact values")
    got = _probe_scores(torch.from_numpy(q8).to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(k8).to(DEV),
                        torch.from_numpy(ks).to(DEV), T)
    for b in range(B):
        ref = O.score_row(q8[b], w[b], k8[b], ks[b], T, T)
        m = np.max(np.abs(ref))
        assert np.max(np.abs(got[b] - ref)) <= 1e-6 * m + 1e-6


def test_fp8_mfma_accuracy_on_the_decode_workload():
    wl = W.WORKLOADS["decode_b16_t16384"]
    inp = W.make_inputs(wl, seed=0)
    g = gpu_pipeline(inp)
    q8 = g.q_fp8.reshape(wl.B, 64, 128)
    w_eff = g.w_eff.reshape(wl.B, 64)
    log("[probe] fp8 MFMA on decode_b16_t16384")
    fp8 = _probe_scores(q8, w_eff, g.cache, g.cache_scale, wl.T)
    f16 = g.scores.reshape(wl.B, wl.T).cpu().numpy()
    oc = OracleCase(inp)
    rows = [0, 5, 10, 15]
    ref = [oc.row(b, 0).scores for b in rows]
    m = max(float(np.max(np.abs(r))) for r in ref)
    e8 = max(float(np.max(np.abs(fp8[b] - r))) for b, r in zip(rows, ref))
    e16 = max(float(np.max(np.abs(f16[b] - r))) for b, r in zip(rows, ref))
    log(f"[probe] max |S - S_ref| / max |S_ref| over rows {rows}: fp8 MFMA {e8 / m:.3e}, "
        f"f16 MFMA (library) {e16 / m:.3e}; bound 1e-5 (+1e-6 absolute)")
    assert e16 <= tol(m)
    assert np.isfinite(e8) and e8 / m < 1e-2          # the probe computes the same scores, coarsely
