"""The library against its LDS-poisoning debug build on the GPU.

liblk_lds_poison.so is the same source built with -DLK_POISON_LDS: every kernel fills
its shared memory with 0xFF bytes (NaN as float32, f16 and e4m3fn) before first use.  A
kernel that read LDS no thread had written would carry that garbage into its outputs,
so on every entry point whose kernels use LDS the two builds must agree bit for bit:
scores, top-k indices, written cache rows, quantized queries, folded weights, and the
sparse MLA output.  The workloads reach each kernel: the fused decode step
(decode_kernel), its ragged many-row form (decode_units_kernel), the one-launch select
(decode_kernel with the top-k in LDS), the separate score calls (decode_pipe_kernel,
and the unit runs on a prepared query), prefill with both grid forms
(score_prefill_kernel), both top-k block shapes, and the sparse MLA split kernel."""
import contextlib
import os

import pytest
import torch

from sparse_attention_lightning_fp8_amd import _lib, build as lkbuild, workloads as W
from tests._parity import gpu_pipeline, gpu_pipeline_fused, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def poisoned():
    lib = _lib.open_library(lkbuild.POISON_LIB_PATH)
    _lib.load()
    return lib


@contextlib.contextmanager
def _using(lib):
    """Route the Python binding through `lib` for the duration of the block."""
    saved = _lib._lib
    _lib._lib = lib
    try:
        yield
    finally:
        _lib._lib = saved


def _same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    if a.is_floating_point():
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b), f"{what} differs between the library and its LDS-poisoned build"


def _compare(r0, r1):
    for name in ("cache", "cache_scale", "q_fp8", "w_eff", "q_scale", "scores", "idx"):
        _same(getattr(r0, name), getattr(r1, name), name)


def _ragged(name, lens, T, k, seed):
    wl = W.Workload(name=name, B=len(lens), S=1, T=T, cap=T + 8, start_pos=-1, k=k, causal=False, ragged=True)
    base = W.make_inputs(wl, seed=seed)
    lt = torch.tensor(lens, dtype=torch.int32)
    return W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))


def _both(poisoned, fn):
    r0 = fn()
    with _using(poisoned):
        r1 = fn()
    return r0, r1


def test_fused_decode_and_select(poisoned):
    """decode_kernel (three key blocks a row), topk_kernel<256>, and lk_decode_select's
    one launch on rows of up to 1001 keys, with and without RoPE."""
    wl = W.Workload(name="poison_decode", B=3, S=1, T=3000, cap=3000, start_pos=2999, k=256, causal=False,
                    ragged=False)
    inp = W.make_inputs(wl, seed=41)
    for rope in (False, True):
        log(f"[poison] fused decode B=3 T=3000 rope={rope}")
        _compare(*_both(poisoned, lambda: gpu_pipeline_fused(inp, rope=rope)))
    sel = _ragged("poison_select", [1, 100, 640, 1001], 1001, 256, seed=42)
    for rope in (False, True):
        log(f"[poison] lk_decode_select rows of 1..1001 keys rope={rope}")
        _compare(*_both(poisoned, lambda: gpu_pipeline_fused(sel, rope=rope, select=True)))


def test_ragged_many_rows(poisoned):
    """64 ragged rows: the unit runs (decode_units_kernel) of the fused step and of the
    separate score on a prepared query, topk_kernel<1024>."""
    inp = W.make_inputs(W.WORKLOADS["ragged_decode_b64"], seed=0)
    log("[poison] ragged_decode_b64 fused step")
    _compare(*_both(poisoned, lambda: gpu_pipeline_fused(inp)))
    log("[poison] ragged_decode_b64 separate calls")
    _compare(*_both(poisoned, lambda: gpu_pipeline(inp)))


def test_separate_decode_and_prefill(poisoned):
    """lk_prepare + lk_index_score + lk_topk: decode_pipe_kernel, score_prefill_kernel
    on 4096-key slices (causal, start_pos, a partial last token group, T not a multiple
    of 64) and on whole-row items (B * ceil(S / 8) >= 2 x the compute units)."""
    cases = [
        W.Workload(name="poison_decode_sep", B=3, S=1, T=3000, cap=3000, start_pos=2999, k=256, causal=False,
                   ragged=False),
        W.Workload(name="poison_prefill", B=1, S=70, T=777, cap=777, start_pos=707, k=128, causal=True,
                   ragged=False),
        W.Workload(name="poison_prefill_whole_row", B=2, S=2053, T=5000, cap=5000, start_pos=2947, k=512,
                   causal=True, ragged=False),
    ]
    for wl in cases:
        inp = W.make_inputs(wl, seed=43)
        log(f"[poison] separate calls {wl.name}: B={wl.B} S={wl.S} T={wl.T}")
        _compare(*_both(poisoned, lambda: gpu_pipeline(inp)))


def test_sparse_mla(poisoned):
    """mla_split_kernel (and the combine) over 2048 selected slots with -1 padding."""
    from sparse_attention_lightning_fp8_amd import api
    wl = W.MlaWorkload("poison_mla", B=2, cap=3000, n_idx=2048)
    inp = W.make_mla_inputs(wl, seed=44)
    idx = inp.idx.clone()
    idx[1, 1500:] = -1
    d = lambda t: t.to(DEV)

    def run():
        out = api.lk_sparse_mla_decode(d(inp.q_lat), d(inp.q_rope), d(inp.kv_lat), d(inp.kv_rope), d(idx),
                                       W.MLA_SCALE)
        torch.cuda.synchronize()
        return out

    log("[poison] sparse MLA B=2 cap=3000 n_idx=2048")
    out0, out1 = _both(poisoned, run)
    _same(out0, out1, "sparse MLA output")
