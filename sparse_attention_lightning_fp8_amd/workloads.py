"""Seeded synthetic inputs shaped like the pages' indexer workloads.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no rotation, quantization, scoring or selection), so both the HIP path
and the CPU oracle can consume the same inputs.

Recipe (one torch CPU generator per tensor, seeded ``16 * seed + stream``):
  * Q: bfloat16 draws of N(0, 1), shape [B, S, 64, 128]          (stream 0)
  * K: bfloat16 draws of N(0, 1), shape [B, cap, 128]            (stream 1)
    -- every cache row a sequence can hold; rows at or beyond a sequence's
       valid length are never read by a correct kernel.
  * w: float32 N(0, 1) / 8, shape [B, S, 64]                     (stream 2)
    -- the per-head weights after the 1/sqrt(64) factor (page "Index scores":
       the 1/sqrt(64) is folded into the weights before the kernel).
  * lens: int32 uniform integers in [1024, 16384], shape [B]     (stream 3, ragged only)
Float draws are float32 ``torch.randn`` rounded to bfloat16 by torch (nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

HEADS = 64
DIM = 128
CAP = 16384


@dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # sequences
    S: int                 # query tokens per sequence in this step
    T: int                 # key slots scored per row (end_pos)
    start_pos: int         # absolute position of query token 0
    cap: int               # cache rows per sequence
    causal: bool           # key s > start_pos + t is masked
    ragged: bool           # per-sequence valid lengths drawn uniform in [1024, 16384]
    k: int                 # top-k size
    note: str = field(default="", compare=False)


# Shapes from the pages: decode at p = 1000 (1001 keys), 64 index heads x 128 dims,
# 16384 cache positions per sequence slot, decode batch 16 (the NKI page's shipping
# shape), plus the prefill / ragged / chunked-prefill cases built from them.
WORKLOADS = {
    "decode_b1_t1001": Workload("decode_b1_t1001", B=1, S=1, T=1001, start_pos=1000, cap=1001,
                                causal=False, ragged=False, k=256,
                                note="decode at position 1000, top-256"),
    "decode_b16_t16384": Workload("decode_b16_t16384", B=16, S=1, T=16384, start_pos=16383,
                                  cap=16384, causal=False, ragged=False, k=2048,
                                  note="decode, 16 sequences, full 16384-slot cache, top-2048"),
    "ragged_decode_b64": Workload("ragged_decode_b64", B=64, S=1, T=16384, start_pos=-1,
                                  cap=16384, causal=False, ragged=True, k=2048,
                                  note="decode, 64 sequences, lengths U[1024,16384], top-min(2048,len)"),
    "prefill_s4096": Workload("prefill_s4096", B=1, S=4096, T=4096, start_pos=0, cap=4096,
                              causal=True, ragged=False, k=2048,
                              note="causal prefill 4096x4096, top-min(2048,t+1)"),
    "chunked_prefill_b2_s4096": Workload("chunked_prefill_b2_s4096", B=2, S=4096, T=16384,
                                         start_pos=12288, cap=16384, causal=True, ragged=False,
                                         k=2048,
                                         note="2 sequences, 4096 new tokens at 12288..16383, top-2048"),
}


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(16 * seed + stream)
    return g


def bf16_normal(shape, seed: int, stream: int) -> torch.Tensor:
    """bfloat16 N(0,1) draws (CPU)."""
    return torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32).to(torch.bfloat16)


def f32_normal_over8(shape, seed: int, stream: int) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32) * 0.125


def lengths(B: int, seed: int, stream: int = 3, lo: int = 1024, hi: int = 16384) -> torch.Tensor:
    return torch.randint(lo, hi + 1, (B,), generator=_gen(seed, stream), dtype=torch.int32)


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor                # bf16 [B, S, H, D]
    k: torch.Tensor                # bf16 [B, cap, D]
    w: torch.Tensor                # f32  [B, S, H]
    lens: Optional[torch.Tensor]   # i32  [B] or None
    positions: torch.Tensor        # i32  [B]: cache row of query token 0 of each sequence


def make_inputs(wl: Workload, seed: int = 0) -> Inputs:
    q = bf16_normal((wl.B, wl.S, HEADS, DIM), seed, 0)
    k = bf16_normal((wl.B, wl.cap, DIM), seed, 1)
    w = f32_normal_over8((wl.B, wl.S, HEADS), seed, 2)
    lens = lengths(wl.B, seed) if wl.ragged else None
    if wl.ragged:
        positions = (lens - wl.S).to(torch.int32)     # the step's tokens end at len - 1
    else:
        positions = torch.full((wl.B,), wl.start_pos, dtype=torch.int32)
    return Inputs(wl, q, k, w, lens, positions)


ROPE_DIM = 64
ROPE_THETA = 10000.0


def rope_tables(positions):
    """cos / sin float32 [n, ROPE_DIM / 2] of plain RoPE angles pos * THETA^(-2i/ROPE_DIM)
    for the given absolute positions (angles in float64, then rounded to float32)."""
    import numpy as np
    inv = ROPE_THETA ** (-np.arange(ROPE_DIM // 2, dtype=np.float64) * 2.0 / ROPE_DIM)
    ang = np.asarray(positions, np.float64).reshape(-1, 1) * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def query_positions(inp: "Inputs"):
    """Absolute position of every query token, [B, S] int64 (token t of sequence b sits
    at positions[b] + t)."""
    import numpy as np
    return inp.positions.numpy().astype(np.int64)[:, None] + np.arange(inp.wl.S, dtype=np.int64)[None, :]


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bfloat16 CPU tensor's bit patterns."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# Sparse MLA decode (page "Join query parts"): 128 heads, 512 latent + 64 rotary
# features, over the 2048 slots the indexer selected out of a 16384-slot cache.
@dataclass(frozen=True)
class MlaWorkload:
    name: str
    B: int
    cap: int
    n_idx: int
    note: str = field(default="", compare=False)


MLA_WORKLOADS = {
    "mla_decode_b16_t16384": MlaWorkload("mla_decode_b16_t16384", B=16, cap=16384, n_idx=2048,
                                         note="16 decode rows, top-2048 of 16384 cached latent rows"),
}
MLA_SCALE = 576 ** -0.5        # the joined 576-feature width of page "Join query parts"


@dataclass
class MlaInputs:
    wl: MlaWorkload
    q_lat: torch.Tensor            # bf16 [B, 128, 512]
    q_rope: torch.Tensor           # bf16 [B, 128, 64]
    kv_lat: torch.Tensor           # bf16 [B, cap, 512]
    kv_rope: torch.Tensor          # bf16 [B, cap, 64]
    idx: torch.Tensor              # i32  [B, n_idx], distinct slots, -1 padding


def mla_indices(B: int, cap: int, n_idx: int, seed: int, lens=None) -> torch.Tensor:
    """Distinct random slots per row (the shape of a top-k set), -1 beyond min(n_idx, len)."""
    g = _gen(seed, 9)
    out = torch.full((B, n_idx), -1, dtype=torch.int32)
    for b in range(B):
        L = cap if lens is None else int(lens[b])
        k = min(n_idx, L)
        if k > 0:
            out[b, :k] = torch.randperm(L, generator=g)[:k].to(torch.int32)
    return out


def make_mla_inputs(wl: MlaWorkload, seed: int = 0, lens=None) -> MlaInputs:
    return MlaInputs(wl, bf16_normal((wl.B, 128, 512), seed, 5), bf16_normal((wl.B, 128, 64), seed, 6),
                     bf16_normal((wl.B, wl.cap, 512), seed, 7), bf16_normal((wl.B, wl.cap, 64), seed, 8),
                     mla_indices(wl.B, wl.cap, wl.n_idx, seed, lens))

