"""Host-side pieces of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
and pair counts its roofline and TFLOP/s figures divide by, and the rule that the
measured-traffic figure is published only for the kernel sources it was taken on."""
import json
import os
import subprocess
import sys

import bench
from sparse_attention_lightning_fp8_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_decode_algorithmic_bytes_c1():
    # 16 rows: 16,383 cached keys x 132 B, the new key 256 B read + 132 B written,
    # 16,384 score slots x 4 B, 64 x 256 B of bf16 query + 64 x 4 B weights, 256 B of
    # RoPE table row
    wl = W.WORKLOADS["decode_b16_t16384"]
    inp = W.make_inputs(wl, seed=0)
    per_row = 16383 * 132 + 256 + 132 + 16384 * 4 + 64 * 256 + 64 * 4 + 256
    assert bench.fused_decode_bytes(wl, inp) == 16 * per_row == 35926016


def test_valid_pairs_causal_prefill():
    # causal, start_pos 0, S = T = 4096: row t has t + 1 valid keys
    wl = W.WORKLOADS["prefill_s4096"]
    inp = W.make_inputs(wl, seed=0)
    assert bench.valid_pairs(wl, inp) == 4096 * 4097 // 2


def test_valid_pairs_chunked_prefill():
    # two sequences, S = 4096 rows from start_pos 12288, T = 16384: row t has 12289 + t keys
    wl = W.WORKLOADS["chunked_prefill_b2_s4096"]
    inp = W.make_inputs(wl, seed=0)
    # (12289 + 16384) / 2 keys on average over 4096 rows (the last row reaches T exactly)
    assert bench.valid_pairs(wl, inp) == 2 * (4096 * 12289 + 4095 * 4096 // 2) == 117444608


def test_traffic_published_only_for_matching_sources(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert bench.measured_traffic() in (None, rec["bytes_per_launch"])
    stale = dict(rec, score_src_sha256="0" * 64)
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() is None
    fresh = dict(rec, score_src_sha256=bench.source_hash())
    f.write_text(json.dumps(fresh))
    assert bench.measured_traffic() == rec["bytes_per_launch"]
