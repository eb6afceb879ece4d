"""lk_decode_score (new key write + query quantization + index score in one launch)
on the GPU against the oracle: the new key's cache bytes and scale, the quantized
query and folded weights bit-exact, scores within 1e-5 max|S_ref| + 1e-6, top-k sets
equal up to swaps at the k-th boundary; and bitwise equal to the unfused path."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightning_fp8_amd import api
from sparse_attention_lightning_fp8_amd import workloads as W
from tests._parity import OracleCase, compare_scores, compare_topk, gpu_pipeline, gpu_pipeline_fused, log, tol

pytestmark = pytest.mark.gpu
DECODE = ["decode_b1_t1001", "decode_b16_t16384", "ragged_decode_b64"]


def _check_against_oracle(inp, g, rows):
    wl = inp.wl
    oc = OracleCase(inp)
    cache = g.cache.cpu().numpy()
    cscale = g.cache_scale.cpu().numpy()
    q8 = g.q_fp8.cpu().numpy().reshape(wl.B, 64, 128)
    we = g.w_eff.cpu().numpy().reshape(wl.B, 64)
    scores = g.scores.cpu().numpy().reshape(wl.B, wl.T)
    idx = g.idx.cpu().numpy().reshape(wl.B, wl.k)
    ref = []
    for b in rows:
        r = oc.row(b, 0)
        ref.append(r)
        oq8, _, ow = oc.query(b, 0)
        assert np.array_equal(q8[b], oq8), f"query bytes differ (b={b})"
        assert np.array_equal(we[b].view(np.uint32), ow.view(np.uint32)), f"folded weights differ (b={b})"
        if r.L >= 1:
            k8, ks = oc.keys(b, r.L)
            assert np.array_equal(cache[b, r.L - 1], k8[r.L - 1]), f"new key bytes differ (b={b}, slot {r.L - 1})"
            assert cscale[b, r.L - 1] == ks[r.L - 1], f"new key scale differs (b={b})"
        assert np.all(cache[b, max(r.L, 0):] == 0xAA), f"bytes written past slot L-1 (b={b})"
    worst = compare_scores([scores[b] for b in rows], ref)
    tau = tol(max(float(np.max(np.abs(r.scores[np.isfinite(r.scores)]), initial=0.0)) for r in ref))
    for b, r in zip(rows, ref):
        compare_topk(idx[b], r, wl.k, tau)
    return worst


@pytest.mark.parametrize("name", DECODE)
def test_fused_decode_workloads(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)
    log(f"[fused] {name}: B={wl.B} T={wl.T}")
    g = gpu_pipeline_fused(inp)
    if inp.lens is not None:                         # 16+ rows: the two shortest, the two longest, every 4th
        order = np.argsort(inp.lens.numpy(), kind="stable")
        rows = sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2])} | set(range(0, wl.B, 4)))
    else:                                            # every row
        rows = list(range(wl.B))
    worst = _check_against_oracle(inp, g, rows)
    log(f"[fused] {name}: worst relative score error {worst:.2e}")


@pytest.mark.parametrize("name", DECODE)
def test_fused_equals_unfused(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=1)
    log(f"[fused] {name} vs lk_prepare + lk_index_score")
    a = gpu_pipeline(inp)
    f = gpu_pipeline_fused(inp)
    sa = a.scores.reshape(wl.B, wl.T)
    sf = f.scores.reshape(wl.B, wl.T)
    assert torch.equal(sa.view(torch.int32), sf.view(torch.int32))
    assert torch.equal(a.q_fp8.reshape(-1), f.q_fp8.reshape(-1))
    assert torch.equal(a.w_eff.reshape(-1).view(torch.int32), f.w_eff.reshape(-1).view(torch.int32))
    assert torch.equal(a.idx.reshape(wl.B, wl.k), f.idx.reshape(wl.B, wl.k))
    for b in range(wl.B):
        sl = int(inp.lens[b]) if inp.lens is not None else -1
        L = O.valid_len(wl.T, sl, wl.causal, wl.start_pos, 0)
        assert torch.equal(a.cache[b, :L], f.cache[b, :L])
        assert torch.equal(a.cache_scale[b, :L], f.cache_scale[b, :L])


def test_fused_ragged_edges():
    """Row lengths at and around the 1024-key block boundary, a single key, no key,
    and T not a multiple of the block: every row checked whole against the oracle."""
    lens = [0, 1, 2, 31, 32, 33, 1023, 1024, 1025, 2047, 2500, 2600]
    wl = W.Workload(name="ragged_edges", B=len(lens), S=1, T=2600, cap=2700, start_pos=-1, k=2048,
                    causal=False, ragged=True)
    base = W.make_inputs(wl, seed=3)
    lt = torch.tensor(lens, dtype=torch.int32)
    inp = W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))
    log("[fused] ragged edge rows")
    g = gpu_pipeline_fused(inp)
    _check_against_oracle(inp, g, list(range(wl.B)))


@pytest.mark.gpu
def test_fused_many_rows_edges():
    """More row blocks than the chip holds at once (130 rows x 3 key blocks), so the
    kernels run as one block per compute unit walking a range of the valid blocks; the
    edge lengths repeat across rows so ranges start and end inside rows, rows with no
    key still return their quantized query, and the fused and separate paths agree."""
    edge = [0, 1, 2, 31, 32, 33, 1023, 1024, 1025, 2047, 2500, 2600, 1500]
    lens = [edge[i % len(edge)] for i in range(130)]
    wl = W.Workload(name="many_rows_edges", B=len(lens), S=1, T=2600, cap=2700, start_pos=-1, k=2048,
                    causal=False, ragged=True)
    base = W.make_inputs(wl, seed=5)
    lt = torch.tensor(lens, dtype=torch.int32)
    inp = W.Inputs(wl, base.q, base.k, base.w, lt, (lt - 1).to(torch.int32))
    log("[fused] 130 rows x 3 key blocks, edge lengths")
    g = gpu_pipeline_fused(inp)
    rows = sorted(set(range(0, 13)) | {13, 40, 64, 77, 100, 116, 127, 128, 129})
    _check_against_oracle(inp, g, rows)
    # the standalone score kernel (same schedule) on the cache and query the fused step left
    sc = api.lk_index_score(g.q_fp8, g.w_eff, g.cache, g.cache_scale, wl.T, seq_len=lt.to("cuda:0"))
    torch.cuda.synchronize()
    assert torch.equal(g.scores.view(torch.int32), sc.view(torch.int32)), "fused and standalone scores differ"


def _new_key_rows(rows_bits: np.ndarray, rope: bool, seed: int):
    """Write each row as the new key of its own one-slot sequence through
    lk_decode_score; return the cache bytes and scales it wrote, and the oracle's."""
    n = rows_bits.shape[0]
    g = torch.Generator().manual_seed(seed)
    dev = "cuda:0"
    q = torch.randn(n, 64, 128, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(n, 64, generator=g) * 0.125).to(dev)
    k_new = torch.from_numpy(rows_bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    cache = torch.full((n, 2, 128), 0xAA, dtype=torch.uint8, device=dev)
    scale = torch.full((n, 2), -1.0, dtype=torch.float32, device=dev)
    tabs = None
    if rope:
        ang = torch.rand(n, 32, generator=g, dtype=torch.float64) * 6.283185307179586
        tabs = (torch.cos(ang).float(), torch.sin(ang).float())
    api.lk_decode_score(q, w, k_new, cache, scale, T=1,
                        rope=None if tabs is None else (tabs[0].to(dev), tabs[1].to(dev)))
    torch.cuda.synchronize()
    if tabs is None:
        oc, os_ = O.quantize_rows(rows_bits)
    else:
        oc, os_ = O.rope_quantize_rows(rows_bits, tabs[0].numpy(), tabs[1].numpy())
    return cache[:, 0].cpu().numpy(), scale[:, 0].cpu().numpy(), oc, os_


@pytest.mark.parametrize("rope", [False, True])
def test_new_key_quantization_many_rows(rope):
    """The new key is quantized by a whole wave (two features a lane); its bytes and
    scale must equal the oracle's on random rows over 2^-20..2^20, on single-value
    rows spanning the bf16 range, and on the edge rows of the quantizer tests.  With
    RoPE the rows stay where the oracle's exact rotation holds (magnitudes within
    2^38 after the rotation): the random rows and single values in [2^-60, 2^60]."""
    g = torch.Generator().manual_seed(7)
    rnd = torch.randn(3000, 128, generator=g) * torch.exp2(torch.randint(-20, 20, (3000, 1), generator=g).float())
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float()
    keep = (torch.isfinite(vals) & (vals.abs() < 2.0**120)).numpy()
    if rope:
        keep &= ((vals.abs() >= 2.0**-60) & (vals.abs() <= 2.0**60)).numpy()
    single = np.zeros((int(keep.sum()) // 4 + 1, 128), np.uint16)
    v = allbits[keep][::4]
    single[:v.size, 5] = v
    single[1::2, 77] = single[1::2, 5]
    f = lambda a: W.bf16_bits(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))
    edge = np.stack([f([0.0] * 128), f([-0.0] * 128), f([1.0] * 128), f([(-1.0) ** i for i in range(128)]),
                     f([448.0 if i == 3 else 0.0 for i in range(128)]), f([2.0**-100] * 64 + [-(2.0**-100)] * 64),
                     f([2.0**60 * (1 + i / 128) for i in range(128)]), f([2.0**-30 if i % 2 else 2.0**8 for i in range(128)]),
                     f([float(i - 64) for i in range(128)]), f([2.0**-126, -(2.0**-133)] + [0.0] * 126)])
    parts = [W.bf16_bits(rnd.to(torch.bfloat16)), single] + ([] if rope else [edge])
    rows = np.concatenate(parts)
    log(f"[fused] new-key quantization, {rows.shape[0]} rows, rope={rope}")
    gc, gs, oc, os_ = _new_key_rows(rows, rope, seed=8)
    bad = np.nonzero(np.any(gc != oc, axis=1) | (gs.view(np.uint32) != os_.view(np.uint32)))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[0]}: gpu {gc[bad[0]][:8]} {gs[bad[0]]} oracle {oc[bad[0]][:8]} {os_[bad[0]]}"
