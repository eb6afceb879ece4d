"""Benchmark of the lightning-indexer hot path on one MI355X.

A step is one pass of the whole path over one batch: RoPE, Hadamard rotation and fp8
quantization of the step's new keys (written to the cache) and of the queries with the
weight fold, fp8 index score with mask, per-row top-k.
Each timed workload first runs its own steps back to back, untimed, for --settle-ms
(300 ms) so the clocks reach their sustained-load state, then --warmup steps.
The step rate comes from an uninstrumented timed loop; per-kernel durations come from a
second pass of the same steps with events recorded at each dispatch's start and end.
The timed workload is decode with 16 sequences of 16384 cached keys (64 heads x 128,
top-2048), run as lk_decode_score (key write + query preparation + score in one
launch) then lk_topk; every input is resident in HBM before timing, and R copies of
the inputs are rotated so the 256 MB last-level cache cannot serve the 33 MB key
cache.  The same step through the separate entry points (lk_prepare, lk_index_score,
lk_topk) is timed too and reported under "extra".

Prints ONE JSON line.  Prefill (4096x4096 causal), chunked prefill (2 x 4096 new
tokens against 16384 keys) and the sparse MLA decode attention over the selected
slots (16 rows, 2048 of 16384) are timed too and reported under "extra".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode keys scored/s + HBM GB/s (B16,T16K); prefill index fp8 TFLOP/s"
HBM_PEAK_GBPS = 8000.0
F16_PEAK_TFLOPS = 2500.0      # dense f16 MFMA (the dtype the contraction runs in)
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0      # dense fp8 MFMA
BYTES_PER_KEY = 136           # 128 B key + 4 B key scale + 4 B score
BYTES_PER_QUERY_ROW = 64 * (128 + 4)
FLOP_PER_PAIR = 2 * 64 * 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SCORE_SRCS = [os.path.join(ROOT, "sparse_attention_lightning_fp8_amd", "csrc", f)
              for f in ("score.hip", "quant_device.h", "lk_device.h", "topk_device.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Seconds of untimed back-to-back steps before each timed workload.  The GPU raises its
# clocks over the first tens of milliseconds of sustained load: timed right after a few
# warmup steps, a decode step measured 18.7-19.0 us and the causal 4096 x 4096 prefill
# score 116 us; after 300 ms of the same steps, 17.5 us and 107 us.
SETTLE_S = 0.3


def settle(step, seconds=None):
    """Run `step()` back to back (synchronizing every 20 calls) for `seconds` of wall time."""
    import torch
    seconds = SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
            n += 1
        torch.cuda.synchronize()
    return n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=16, help="input copies cycled through to defeat the LLC")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-mla", action="store_true")
    ap.add_argument("--no-ragged", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back steps of each workload, in ms of wall time, before its "
                         "warmup and timed steps (lets the clocks reach their sustained-load state)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the two prefill workloads (for profiling runs); prints no JSON line")
    ap.add_argument("--floors-only", action="store_true",
                    help="only the probe-kernel floors (empty launch, plain read); prints no JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    return ap.parse_args()


# ---------------------------------------------------------------------------- setup
class DecodeSet:
    """One copy of every input and output of a decode step."""

    def __init__(self, api, inp, cache, cache_scale, dev):
        import torch
        wl = inp.wl
        self.cache = cache
        self.cache_scale = cache_scale
        self.k_new = torch.stack([inp.k[b, int(inp.positions[b]):int(inp.positions[b]) + wl.S]
                                  for b in range(wl.B)]).to(dev)
        self.positions = inp.positions.to(dev)
        self.q = inp.q.to(dev)
        self.w = inp.w.to(dev)
        self.q8 = torch.empty(self.q.shape, dtype=torch.uint8, device=dev)
        self.w_eff = torch.empty_like(self.w)
        self.scores = torch.empty((wl.B, wl.S, wl.T), dtype=torch.float32, device=dev)
        self.idx = torch.empty((wl.B, wl.S, wl.k), dtype=torch.int32, device=dev)
        self.seq_len = inp.lens.to(dev) if inp.lens is not None else None
        # RoPE tables of the step's tokens (the new keys sit at the query positions)
        from sparse_attention_lightning_fp8_amd import workloads as W
        c, s = W.rope_tables(W.query_positions(inp).reshape(-1))
        self.rope_tabs = (torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev))
        self.k_rope = self.q_rope = (self.rope_tabs[0].data_ptr(), self.rope_tabs[1].data_ptr())


def make_sets(api, inp, n_sets, dev):
    import torch
    wl = inp.wl
    cache = torch.zeros((wl.B, wl.cap, 128), dtype=torch.uint8, device=dev)
    cache_scale = torch.zeros((wl.B, wl.cap), dtype=torch.float32, device=dev)
    api.lk_quantize_keys(inp.k.to(dev), cache, cache_scale)      # the cached prefix (untimed)
    sets = [DecodeSet(api, inp, cache, cache_scale, dev)]
    for _ in range(n_sets - 1):
        sets.append(DecodeSet(api, inp, cache.clone(), cache_scale.clone(), dev))
    torch.cuda.synchronize()
    return sets


def raw_calls(wl, s):
    """Pre-marshalled C-ABI calls of one step (the same entry points the Python binding
    wraps, with the argument checks done once), so the host enqueues a step in a few
    microseconds and the GPU, not Python, sets the pace of the timed loop."""
    import ctypes
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    cap = s.cache.shape[1]
    seq_len = s.seq_len.data_ptr() if s.seq_len is not None else None
    s.rows = _lib.LkRows(wl.B, wl.S, wl.T, wl.start_pos, seq_len, 1 if wl.causal else 0)
    rows = ctypes.byref(s.rows)
    return [
        (lib.lk_prepare, (s.k_new.data_ptr(), wl.B, wl.S, s.k_new.stride(0) // 128, s.cache.data_ptr(),
                          s.cache_scale.data_ptr(), cap, cap, 0, s.positions.data_ptr(),
                          s.q.data_ptr(), s.w.data_ptr(), wl.B * wl.S, 64, s.q8.data_ptr(),
                          s.w_eff.data_ptr(), None, s.k_rope[0], s.k_rope[1], s.q_rope[0], s.q_rope[1], stream)),
        (lib.lk_index_score, (s.q8.data_ptr(), s.w_eff.data_ptr(), 64, s.cache.data_ptr(), s.cache_scale.data_ptr(),
                              cap, rows, s.scores.data_ptr(), stream)),
        (lib.lk_topk, (s.scores.data_ptr(), rows, wl.k, s.idx.data_ptr(), stream)),
    ]


def raw_calls_fused(wl, s):
    """The same step as raw_calls through lk_decode_score + lk_topk (decode rows only)."""
    import ctypes
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    cap = s.cache.shape[1]
    seq_len = s.seq_len.data_ptr() if s.seq_len is not None else None
    s.rows = _lib.LkRows(wl.B, wl.S, wl.T, wl.start_pos, seq_len, 1 if wl.causal else 0)
    rows = ctypes.byref(s.rows)
    return [
        (lib.lk_decode_score, (s.q.data_ptr(), s.w.data_ptr(), 64, s.k_new.data_ptr(), s.cache.data_ptr(),
                               s.cache_scale.data_ptr(), cap, rows, s.scores.data_ptr(), None, None,
                               s.q_rope[0], s.q_rope[1], stream)),
        (lib.lk_topk, (s.scores.data_ptr(), rows, wl.k, s.idx.data_ptr(), stream)),
    ]


def raw_calls_select(wl, s, keep_scores=True):
    """The same step as raw_calls_fused through one lk_decode_select call (one launch for
    rows of at most 1024 keys; no score written unless keep_scores)."""
    import ctypes
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    cap = s.cache.shape[1]
    seq_len = s.seq_len.data_ptr() if s.seq_len is not None else None
    s.rows = _lib.LkRows(wl.B, wl.S, wl.T, wl.start_pos, seq_len, 1 if wl.causal else 0)
    rows = ctypes.byref(s.rows)
    return [
        (lib.lk_decode_select, (s.q.data_ptr(), s.w.data_ptr(), 64, s.k_new.data_ptr(), s.cache.data_ptr(),
                                s.cache_scale.data_ptr(), cap, rows, s.scores.data_ptr() if keep_scores else None,
                                None, None, s.q_rope[0], s.q_rope[1], wl.k, s.idx.data_ptr(), stream)),
    ]


def run_step(calls, ev=None, arm=None):
    """One pass of the hot path (lk_prepare: key write + query quantize and weight fold;
    lk_index_score; lk_topk).  `ev` (optional) holds one (start, stop) event pair per
    kernel, armed through lk_profile_next_launch so the runtime records them at the
    kernel's own start and end."""
    for j, (fn, args) in enumerate(calls):
        if ev:
            arm(ev[j][0].cuda_event, ev[j][1].cuda_event)
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{fn.__name__} returned {st}")


def make_event_pairs(n_steps, n_kernels):
    import torch
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_kernels)] for _ in range(n_steps)]
    for step in evs:                      # create the HIP events (torch creates them on first record)
        for a, b in step:
            a.record()
            b.record()
    torch.cuda.synchronize()
    return evs


def time_workload(api, wl_name, steps, warmup, n_sets, dev, fused=False, select=None):
    """Warm up, then time `steps` uninstrumented steps (wall clock between two device
    synchronizations: this gives the step rate), then run the same `steps` again with
    dispatch events armed on every kernel (this gives each kernel's mean duration).
    `fused` runs the decode step as lk_decode_score + lk_topk; `select` ("scores" or
    "no_scores") as one lk_decode_select call (rows of at most 1024 keys: one launch)."""
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    from sparse_attention_lightning_fp8_amd import workloads as W
    wl = W.WORKLOADS[wl_name]
    inp = W.make_inputs(wl, seed=0)
    sets = make_sets(api, inp, n_sets, dev)
    if select:
        calls = [raw_calls_select(wl, s, keep_scores=select == "scores") for s in sets]
    else:
        calls = [(raw_calls_fused if fused else raw_calls)(wl, s) for s in sets]
    arm = _lib.load().lk_profile_next_launch
    if select:
        names = ["decode_select"]
    else:
        names = ["decode_score", "topk"] if fused else ["prepare", "index_score", "topk"]
    # the events exist before the settle phase: creating them leaves the GPU idle long
    # enough for its clocks to drop again
    evs = make_event_pairs(steps, len(names))
    it = iter(range(1 << 62))
    settle(lambda: run_step(calls[next(it) % n_sets]))
    for i in range(warmup):
        run_step(calls[i % n_sets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(calls[i % n_sets])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        run_step(calls[i % n_sets], evs[i], arm)
    torch.cuda.synchronize()
    per = {n: sum(e[j][0].elapsed_time(e[j][1]) for e in evs) / steps * 1e3 for j, n in enumerate(names)}
    return wl, inp, wall, per


def fused_decode_bytes(wl, inp):
    """Bytes lk_decode_score must move for one step: per row, the cached keys [0, L-1)
    with their scales (132 B each), the new key (256 B of bf16 read, 132 B written),
    every score slot (4 B), the bf16 query with its weights (64 x 256 B + 64 x 4 B) and
    the token's RoPE tables (2 x 32 x 4 B)."""
    tot = 0
    for b in range(wl.B):
        L = min(wl.T, int(inp.lens[b])) if inp.lens is not None else wl.T
        if wl.causal:
            L = min(L, wl.start_pos + 1)
        L = max(L, 0)
        tot += max(L - 1, 0) * 132 + (256 + 132 if L >= 1 else 0) + wl.T * 4 + 64 * 128 * 2 + 64 * 4 + 256
    return tot


def valid_pairs(wl, inp):
    """Unmasked (query, key) pairs of one step: row (b, t) has
    L = min(T, len_b, start_pos + t + 1 if causal) valid keys."""
    tot = 0
    for b in range(wl.B):
        cap = min(wl.T, int(inp.lens[b])) if inp.lens is not None else wl.T
        for t in range(wl.S):
            L = min(cap, wl.start_pos + t + 1) if wl.causal else cap
            tot += max(L, 0)
    return tot


def time_prefill(api, steps, dev):
    """Prefill (4096 x 4096 causal) and chunked prefill (2 x 4096 new tokens at
    12288..16383 against 16384 keys) through lk_prepare, lk_index_score, lk_topk."""
    import torch
    res = {}
    for name in ("prefill_s4096", "chunked_prefill_b2_s4096"):
        log(f"{name}: setting up")
        pwl, pinp, pwall, pper = time_workload(api, name, steps, 2, 1, dev)
        pairs = valid_pairs(pwl, pinp)
        flops = pairs * FLOP_PER_PAIR
        tf = flops / (pper["index_score"] * 1e-6) / 1e12
        res[name] = {"step_ms": pwall / steps * 1e3, "kernel_us": pper,
                     "valid_pairs": pairs, "score_TFLOPs": tf,
                     "score_frac_f16_peak": tf / F16_PEAK_TFLOPS, "score_frac_fp8_peak": tf / FP8_PEAK_TFLOPS}
        log(f"{name}: score {pper['index_score']:.1f} us = {tf:.1f} TFLOP/s")
        del pinp
        torch.cuda.empty_cache()
    return res


def time_mla(api, steps, warmup, n_sets, dev):
    """Sparse MLA decode over the 2048 selected slots of 16 rows (16384-slot latent
    cache).  n_sets copies of the caches and index lists (seeded, generated on the GPU)
    are rotated so the last-level cache cannot hold the gathered rows."""
    import ctypes
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    from sparse_attention_lightning_fp8_amd import workloads as W
    wl = W.MLA_WORKLOADS["mla_decode_b16_t16384"]
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = lib.lk_sparse_mla_workspace_size(wl.B, wl.n_idx)
    sets = []
    for i in range(n_sets):
        g = torch.Generator(device=dev).manual_seed(1000 + i)
        s = {
            "ql": torch.randn((wl.B, 128, 512), generator=g, device=dev).to(torch.bfloat16),
            "qr": torch.randn((wl.B, 128, 64), generator=g, device=dev).to(torch.bfloat16),
            "kl": torch.randn((wl.B, wl.cap, 512), generator=g, device=dev).to(torch.bfloat16),
            "kr": torch.randn((wl.B, wl.cap, 64), generator=g, device=dev).to(torch.bfloat16),
            "idx": torch.stack([torch.randperm(wl.cap, generator=g, device=dev)[:wl.n_idx]
                                for _ in range(wl.B)]).to(torch.int32),
            "out": torch.empty((wl.B, 128, 512), dtype=torch.float32, device=dev),
            "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
        }
        s["call"] = (s["ql"].data_ptr(), s["qr"].data_ptr(), s["kl"].data_ptr(), s["kr"].data_ptr(), wl.cap, wl.cap,
                     s["idx"].data_ptr(), wl.B, wl.n_idx, ctypes.c_float(W.MLA_SCALE), s["out"].data_ptr(),
                     s["ws"].data_ptr(), ws_bytes, stream)
        sets.append(s)
    fn = lib.lk_sparse_mla_decode
    evs = make_event_pairs(steps, 1)
    it = iter(range(1 << 62))
    settle(lambda: fn(*sets[next(it) % n_sets]["call"]))
    for i in range(warmup):
        fn(*sets[i % n_sets]["call"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st = fn(*sets[i % n_sets]["call"])
        if st != 0:
            raise RuntimeError(f"lk_sparse_mla_decode returned {st}")
    torch.cuda.synchronize()
    call_us = (time.perf_counter() - t0) / steps * 1e6
    for i in range(steps):
        lib.lk_profile_next_launch(evs[i][0][0].cuda_event, evs[i][0][1].cuda_event)
        fn(*sets[i % n_sets]["call"])
    torch.cuda.synchronize()
    split_us = sum(e[0][0].elapsed_time(e[0][1]) for e in evs) / steps * 1e3
    n_sel = wl.B * wl.n_idx
    gathered = n_sel * (512 + 64) * 2
    algo = gathered + wl.B * 128 * (512 + 64) * 2 + wl.B * 128 * 512 * 4 + wl.B * wl.n_idx * 4
    flops = n_sel * 128 * ((512 + 64) + 512) * 2
    return {"call_us": call_us, "split_kernel_us": split_us, "algorithmic_bytes": algo, "flop": flops,
            "hbm_GBps": algo / (call_us * 1e-6) / 1e9, "hbm_frac": algo / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "TFLOPs": flops / (call_us * 1e-6) / 1e12,
            "bf16_mfma_frac": flops / (call_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            "workspace_bytes": ws_bytes, "rotated_input_copies": n_sets}


# ---------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wl_name, seconds=5.0):
    """The oracle (plain single-threaded C through ctypes, which releases the GIL during
    each call) on the same decode step: key write of the new rows, query quantize +
    fold, scores against every cached key, sort-based top-k.  Timed twice on whole steps
    repeated for about `seconds` each: on one core, and with the step's rows split over
    P = min(cpu count, 16) threads, one row range each.  Then the oracle's prefill rate
    (GFLOP/s, 16,384 flop per scored pair) on a sample of chunked-prefill rows over the
    same P threads.  The cache prefix is quantized by the oracle beforehand (untimed)."""
    import concurrent.futures
    import numpy as np
    from oracle import oracle as O
    from sparse_attention_lightning_fp8_amd import workloads as W
    wl = W.WORKLOADS[wl_name]
    inp = W.make_inputs(wl, seed=0)
    P = max(1, min(os.cpu_count() or 1, 16))
    prefix = []
    for b in range(wl.B):
        p0 = int(inp.positions[b])
        prefix.append(O.quantize_rows(W.bf16_bits(inp.k[b, :p0])))

    def rows_step(bs):
        for b in bs:
            p0 = int(inp.positions[b])
            kn, ksn = O.quantize_rows(W.bf16_bits(inp.k[b, p0:p0 + wl.S]))
            k8 = np.concatenate([prefix[b][0], kn])
            ks = np.concatenate([prefix[b][1], ksn])
            for t in range(wl.S):
                q8, qs = O.quantize_rows(W.bf16_bits(inp.q[b, t]))
                w_eff = O.fold_weights(inp.w[b, t].numpy(), qs)
                L = O.valid_len(wl.T, -1, wl.causal, wl.start_pos, t)
                s = O.score_row(q8, w_eff, k8, ks, wl.T, L)
                O.topk(s, L, wl.k)

    def timed(step):
        t0 = time.perf_counter()
        reps = 0
        while reps < 30 and (reps == 0 or time.perf_counter() - t0 < seconds):
            step()
            reps += 1
        return reps, time.perf_counter() - t0

    keys = wl.B * wl.S * wl.T
    reps1, dt1 = timed(lambda: rows_step(range(wl.B)))
    shards = [list(range(wl.B))[i::P] for i in range(P)]
    shards = [s_ for s_ in shards if s_]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(shards)) as ex:
        repsP, dtP = timed(lambda: list(ex.map(rows_step, shards)))
        # prefill: oracle scores of chunked_prefill_b2_s4096 rows (keys written by the oracle)
        pw = W.WORKLOADS["chunked_prefill_b2_s4096"]
        pinp = W.make_inputs(pw, seed=0)
        pk8, pks = O.quantize_rows(W.bf16_bits(pinp.k[0]))
        sample = list(range(0, pw.S, pw.S // (2 * P)))[:2 * P]

        def prow(t):
            q8, qs = O.quantize_rows(W.bf16_bits(pinp.q[0, t]))
            w_eff = O.fold_weights(pinp.w[0, t].numpy(), qs)
            L = O.valid_len(pw.T, -1, pw.causal, pw.start_pos, t)
            O.score_row(q8, w_eff, pk8, pks, pw.T, L)
            return L

        t0 = time.perf_counter()
        pairs = sum(ex.map(prow, sample))
        dtp = time.perf_counter() - t0
    return {"value": keys * repsP / dtP, "unit": "keys/s", "cores": len(shards), "kind": "oracle",
            "sample": f"{repsP} full {wl_name} steps (B={wl.B}, T={wl.T}: key write, query quantize, {keys} key "
                      f"scores, top-{wl.k} each) with the rows split over {len(shards)} threads, {dtP:.2f} s",
            "single_core_keys_per_s": keys * reps1 / dt1,
            "single_core_sample": f"{reps1} steps on one thread, {dt1:.2f} s",
            "prefill_GFLOPs": pairs * FLOP_PER_PAIR / dtp / 1e9,
            "prefill_sample": f"{len(sample)} rows of chunked_prefill_b2_s4096 (sequence 0, {pairs} scored pairs) "
                              f"over {len(shards)} threads, {dtp:.2f} s"}


def probe_floors(dev, launches=200):
    """Floors measured with the library's probe kernels: the duration of an empty kernel
    between its own start and end events (and the wall time per launch back to back),
    and a plain read of the decode workload's 32 MiB key cache, 16 rotated copies (so
    the 256 MB last-level cache cannot serve them), at 1024 and 512 blocks."""
    import torch
    from sparse_attention_lightning_fp8_amd import _lib
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    arm = lib.lk_profile_next_launch
    res = {}
    ev = make_event_pairs(launches, 1)
    for i in range(20):
        lib.lk_probe_empty(256, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(launches):
        lib.lk_probe_empty(256, stream)
    torch.cuda.synchronize()
    res["empty_kernel_wall_us_per_launch"] = (time.perf_counter() - t0) / launches * 1e6
    for i in range(launches):
        arm(ev[i][0][0].cuda_event, ev[i][0][1].cuda_event)
        lib.lk_probe_empty(256, stream)
    torch.cuda.synchronize()
    res["empty_kernel_event_us"] = sum(e[0][0].elapsed_time(e[0][1]) for e in ev) / launches * 1e3
    n = 16384 * 16 * 128                                   # the key cache of decode_b16_t16384
    bufs = [torch.ones(n // 4, dtype=torch.int32, device=dev) for _ in range(16)]
    for blocks in (1024, 512):
        sink = torch.empty(blocks * 4, dtype=torch.int32, device=dev)
        for i in range(20):
            lib.lk_probe_read(bufs[i % 16].data_ptr(), n, sink.data_ptr(), blocks, stream)
        torch.cuda.synchronize()
        for i in range(launches):
            arm(ev[i][0][0].cuda_event, ev[i][0][1].cuda_event)
            lib.lk_probe_read(bufs[i % 16].data_ptr(), n, sink.data_ptr(), blocks, stream)
        torch.cuda.synchronize()
        us = sum(e[0][0].elapsed_time(e[0][1]) for e in ev) / launches * 1e3
        res[f"read_32MiB_{blocks}_blocks_us"] = us
        res[f"read_32MiB_{blocks}_blocks_GBps"] = n / (us * 1e-6) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return res


def empirical_ceilings(dev):
    """Second denominators measured with library kernels (PyTorch's own): a 32 MiB
    device copy (bytes read plus bytes written) and a dense f16 GEMM (8192^3 through
    torch.matmul).  Sixteen copies are rotated so the 256 MB last-level cache does not
    serve them.  (torch.sum over the same 32 MiB reads at under 2 TB/s, a property of
    its reduction, so it is not used as a read ceiling.)"""
    import torch
    n = 32 << 20
    xs = [torch.ones(n // 4, dtype=torch.float32, device=dev) for _ in range(16)]
    ys = [torch.empty_like(x) for x in xs]

    def timed(fn, iters):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters              # us per call

    cp_us = timed(lambda i: ys[i % 16].copy_(xs[i % 16]), 100)
    del xs, ys
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.float16)
    bm = torch.randn(m, m, device=dev, dtype=torch.float16)
    mm_us = timed(lambda i: torch.matmul(a, bm), 10)
    del a, bm
    torch.cuda.empty_cache()
    return {"copy_32MiB_GBps": 2 * n / (cp_us * 1e3), "copy_kernel": "Tensor.copy_ (bytes read + written)",
            "f16_gemm_TFLOPs": 2 * m ** 3 / (mm_us * 1e-6) / 1e12, "gemm": "torch.matmul f16 8192^3"}


# ---------------------------------------------------------------------------- traffic
def source_hash():
    """sha256 over the sources the decode score kernel is built from."""
    h = hashlib.sha256()
    for f in SCORE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per score launch from committed rocprofv3 PMC runs, if they were taken
    on the current score kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = source_hash()
        if rec.get("score_src_sha256") == h:
            return rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


# ---------------------------------------------------------------------------- main
def main():
    args = parse()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle_ms) / 1e3
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the indexer shards by "
              "sequence or query rows with no exchange, so per-GPU throughput is the single-GPU figure.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return
    from sparse_attention_lightning_fp8_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    from sparse_attention_lightning_fp8_amd import api
    dev = "cuda:0"
    torch.cuda.init()

    if args.prefill_only:
        log(json.dumps(time_prefill(api, args.prefill_steps, dev)))
        return
    if args.floors_only:
        log(json.dumps(probe_floors(dev)))
        return

    log("decode_b16_t16384: setting up")
    _, _, uwall, uper = time_workload(api, "decode_b16_t16384", args.steps, args.warmup, args.rotate, dev)
    torch.cuda.empty_cache()
    wl, inp, wall, per = time_workload(api, "decode_b16_t16384", args.steps, args.warmup, args.rotate, dev,
                                       fused=True)
    keys = wl.B * wl.S * wl.T
    ms_step = wall / args.steps * 1e3
    value = keys * args.steps / wall
    score_bytes = fused_decode_bytes(wl, inp)
    score_us = per["decode_score"]
    achieved = score_bytes / (score_us * 1e-6) / 1e9
    log(f"decode (fused): {ms_step * 1e3:.1f} us/step, kernels {per}")
    u_bytes = keys * BYTES_PER_KEY + wl.B * wl.S * BYTES_PER_QUERY_ROW
    log(f"decode (separate calls): {uwall / args.steps * 1e6:.1f} us/step, kernels {uper}")

    extra = {"score_kernel_us": score_us, "score_hbm_GBps": achieved,
             "step_kernel_us": per, "keys_per_s_score_kernel": keys / (score_us * 1e-6),
             "separate_calls": {"step_us": uwall / args.steps * 1e6, "kernel_us": uper,
                                "index_score_hbm_GBps": u_bytes / (uper["index_score"] * 1e-6) / 1e9,
                                "index_score_algorithmic_bytes": u_bytes}}
    if not args.no_ragged:
        # ragged decode (64 rows, lengths uniform in [1024, 16384]) through the fused step
        log("ragged_decode_b64: setting up")
        torch.cuda.empty_cache()
        rwl, rinp, rwall, rper = time_workload(api, "ragged_decode_b64", args.steps, args.warmup, 8, dev, fused=True)
        rbytes = fused_decode_bytes(rwl, rinp)
        rgbps = rbytes / (rper["decode_score"] * 1e-6) / 1e9
        extra["ragged_decode_b64"] = {"step_us": rwall / args.steps * 1e6, "kernel_us": rper,
                                      "algorithmic_bytes": rbytes, "decode_score_hbm_GBps": rgbps,
                                      "decode_score_hbm_frac": rgbps / HBM_PEAK_GBPS,
                                      "valid_keys": valid_pairs(rwl, rinp), "rotated_input_copies": 8}
        log(f"ragged_decode_b64: decode_score {rper['decode_score']:.1f} us = {rgbps:.0f} GB/s")
        del rinp
        torch.cuda.empty_cache()
    # the pages' stated decode step (one sequence at position 1000: 1001 keys, top-256):
    # two launches (lk_decode_score + lk_topk) against one lk_decode_select launch
    log("decode_b1_t1001: setting up")
    torch.cuda.empty_cache()
    swl, _, s2wall, s2per = time_workload(api, "decode_b1_t1001", args.steps, args.warmup, args.rotate, dev,
                                          fused=True)
    _, _, s1wall, s1per = time_workload(api, "decode_b1_t1001", args.steps, args.warmup, args.rotate, dev,
                                        select="scores")
    _, _, s0wall, s0per = time_workload(api, "decode_b1_t1001", args.steps, args.warmup, args.rotate, dev,
                                        select="no_scores")
    extra["decode_b1_t1001"] = {"two_launch_step_us": s2wall / args.steps * 1e6, "two_launch_kernel_us": s2per,
                                "select_step_us": s1wall / args.steps * 1e6, "select_kernel_us": s1per,
                                "select_no_scores_step_us": s0wall / args.steps * 1e6,
                                "select_no_scores_kernel_us": s0per}
    log(f"decode_b1_t1001: two launches {s2wall / args.steps * 1e6:.1f} us/step, lk_decode_select "
        f"{s1wall / args.steps * 1e6:.1f} us/step ({s0wall / args.steps * 1e6:.1f} without scores)")
    torch.cuda.empty_cache()
    if not args.no_prefill:
        extra.update(time_prefill(api, args.prefill_steps, dev))

    if not args.no_mla:
        log("mla_decode_b16_t16384: setting up")
        extra["mla_decode_b16_t16384"] = time_mla(api, args.steps, args.warmup, 4, dev)
        log(f"sparse MLA decode: {extra['mla_decode_b16_t16384']['call_us']:.1f} us per call")
        torch.cuda.empty_cache()

    log("floors (probe kernels): running")
    extra["floors"] = probe_floors(dev)
    log(f"floors: {extra['floors']}")
    log("empirical ceilings: running")
    extra["empirical_ceilings"] = empirical_ceilings(dev)
    log(f"empirical ceilings: {extra['empirical_ceilings']}")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): running")
        cpu = cpu_baseline("decode_b16_t16384")
        log(f"cpu baseline: {cpu['value']:.3e} keys/s on {cpu['cores']} threads, "
            f"{cpu['single_core_keys_per_s']:.3e} on one; prefill {cpu['prefill_GFLOPs']:.2f} GFLOP/s")

    out = {
        "metric": METRIC, "value": value, "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 operands, f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": "decode_b16_t16384", "B": wl.B, "T": wl.T, "heads": 64, "dim": 128,
                   "topk": wl.k, "rotated_input_copies": args.rotate, "settle_ms": args.settle_ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "kernel": "decode_kernel<false> (lk_decode_score)", "algorithmic_bytes": score_bytes},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
