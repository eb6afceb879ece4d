"""Python binding of the lightning-indexer C ABI (include/lk.h).

Each function checks dtypes, shapes and devices of its torch tensors, allocates
outputs the caller did not pass, and forwards pointers, sizes and the current HIP
stream to the C entry point of the same name.  All computation happens in liblk's
kernels; there is no CPU path.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import LkRows

DIM = 128
HEADS = 64
ROPE_DIM = 64


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _byte_view(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _rows(B: int, S: int, T: int, start_pos: int, seq_len: Optional[torch.Tensor], causal: bool) -> LkRows:
    ptr = None
    if seq_len is not None:
        _need(seq_len.dtype == torch.int32 and seq_len.is_cuda and seq_len.is_contiguous()
              and seq_len.numel() >= B, "seq_len must be a contiguous int32 CUDA tensor with B entries")
        ptr = seq_len.data_ptr()
    return LkRows(B, S, T, start_pos, ptr, 1 if causal else 0)


def _key_args(x, cache, cache_scale, row_offset, positions):
    _need(x.dtype == torch.bfloat16 and x.dim() == 3 and x.shape[2] == DIM, "x must be bf16 [n_seq, n_rows, 128]")
    _need(x.stride(2) == 1 and x.stride(1) == DIM and x.stride(0) % DIM == 0, "x rows must be contiguous")
    cache = _byte_view(cache)
    _need(cache.dtype == torch.uint8 and cache.dim() == 3 and cache.shape[2] == DIM
          and cache.stride(2) == 1 and cache.stride(1) == DIM and cache.stride(0) % DIM == 0,
          "cache must be uint8/e4m3fn [N, cap, 128] with contiguous rows")
    cs = cache_scale.squeeze(-1) if cache_scale.dim() == 3 else cache_scale
    seq_stride = cache.stride(0) // DIM
    _need(cs.dtype == torch.float32 and cs.dim() == 2 and cs.shape[:2] == cache.shape[:2]
          and cs.stride(1) == 1 and (cs.shape[0] == 1 or cs.stride(0) == seq_stride),
          "cache_scale must be float32 [N, cap] sharing the cache's sequence stride")
    _need(x.shape[0] <= cache.shape[0], "more sequences than cache slots")
    _need(x.is_cuda and cache.device == x.device and cs.device == x.device, "tensors must be on one CUDA device")
    pos_ptr = None
    if positions is not None:
        _need(positions.dtype == torch.int32 and positions.is_cuda and positions.is_contiguous()
              and positions.numel() >= x.shape[0], "positions must be int32 CUDA [n_seq]")
        pos_ptr = positions.data_ptr()
    return (x.data_ptr(), x.shape[0], x.shape[1], x.stride(0) // DIM, cache.data_ptr(), cs.data_ptr(),
            seq_stride, cache.shape[1], row_offset, pos_ptr)


def _query_args(q, w, q_fp8, w_eff, q_scale):
    _need(q.dtype == torch.bfloat16 and q.shape[-1] == DIM and q.is_contiguous(), "q must be contiguous bf16 [..., H, 128]")
    _need(w.dtype == torch.float32 and w.shape == q.shape[:-1] and w.is_contiguous(), "w must be contiguous float32 [..., H]")
    H = q.shape[-2]
    n_tok = q.numel() // (H * DIM) if H > 0 else 0
    if q_fp8 is None:
        q_fp8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    if w_eff is None:
        w_eff = torch.empty(w.shape, dtype=torch.float32, device=q.device)
    q8 = _byte_view(q_fp8)
    _need(q8.shape == q.shape and q8.is_contiguous() and w_eff.shape == w.shape and w_eff.is_contiguous(),
          "output shapes must match the inputs")
    qs_ptr = None
    if q_scale is not None:
        _need(q_scale.dtype == torch.float32 and q_scale.shape == w.shape and q_scale.is_contiguous(), "bad q_scale")
        qs_ptr = q_scale.data_ptr()
    return (q.data_ptr(), w.data_ptr(), n_tok, H, q8.data_ptr(), w_eff.data_ptr(), qs_ptr), q_fp8, w_eff


def lk_quantize_keys(x: torch.Tensor, cache: torch.Tensor, cache_scale: torch.Tensor,
                     row_offset: int = 0, positions: Optional[torch.Tensor] = None) -> None:
    """Rotate + quantize x [n_seq, n_rows, 128] (bf16) into cache [N, cap, 128] (uint8 or
    float8_e4m3fn) and cache_scale [N, cap] or [N, cap, 1] (float32), rows starting at
    `row_offset` or at positions[b] (int32 CUDA [n_seq])."""
    args = _key_args(x, cache, cache_scale, row_offset, positions)
    _lib.check("lk_quantize_keys", _lib.load().lk_quantize_keys(*args, _stream(x)))


def lk_quantize_queries(q: torch.Tensor, w: torch.Tensor, q_fp8: Optional[torch.Tensor] = None,
                        w_eff: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None):
    """q [..., H, 128] bf16 and w [..., H] float32 -> (q_fp8 uint8 [..., H, 128], w_eff float32 [..., H]).
    If `q_scale` (float32 [..., H]) is given it receives the per-head scales."""
    args, q_fp8, w_eff = _query_args(q, w, q_fp8, w_eff, q_scale)
    _lib.check("lk_quantize_queries", _lib.load().lk_quantize_queries(*args, _stream(q)))
    return q_fp8, w_eff


def _rope_args(rope, n_rows: int, dev):
    """(cos, sin) float32 [n_rows, 32] CUDA tables, or None -> two NULL pointers."""
    if rope is None:
        return None, None
    c, s = rope
    for t in (c, s):
        _need(t.dtype == torch.float32 and t.is_cuda and t.device == dev and t.is_contiguous()
              and t.numel() == n_rows * (ROPE_DIM // 2), f"RoPE tables must be contiguous float32 [{n_rows}, 32]")
    return c.data_ptr(), s.data_ptr()


def lk_prepare(x: torch.Tensor, cache: torch.Tensor, cache_scale: torch.Tensor, q: torch.Tensor,
               w: torch.Tensor, row_offset: int = 0, positions: Optional[torch.Tensor] = None,
               q_fp8: Optional[torch.Tensor] = None, w_eff: Optional[torch.Tensor] = None,
               q_scale: Optional[torch.Tensor] = None, k_rope=None, q_rope=None):
    """lk_quantize_keys + lk_quantize_queries in one kernel launch; returns (q_fp8, w_eff).
    Optional RoPE before the rotation: k_rope = (cos, sin) float32 [n_seq * n_rows, 32]
    (one row per key row), q_rope = (cos, sin) float32 [n_tokens, 32]."""
    kargs = _key_args(x, cache, cache_scale, row_offset, positions)
    qargs, q_fp8, w_eff = _query_args(q, w, q_fp8, w_eff, q_scale)
    _need(q.device == x.device, "tensors must be on one CUDA device")
    kc, ks = _rope_args(k_rope, x.shape[0] * x.shape[1], x.device)
    H = q.shape[-2]
    qc, qs = _rope_args(q_rope, q.numel() // (H * DIM) if H > 0 else 0, x.device)
    _lib.check("lk_prepare", _lib.load().lk_prepare(*kargs, *qargs, kc, ks, qc, qs, _stream(x)))
    return q_fp8, w_eff


def lk_index_score(q_fp8: torch.Tensor, w_eff: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor,
                   T: int, start_pos: int = 0, seq_len: Optional[torch.Tensor] = None, causal: bool = False,
                   scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Masked fp8 index scores [B, S, T] (float32) of q_fp8 [B, S, 64, 128] against keys
    [0, T) of k_cache [>=B, cap, 128] with scales k_scale [>=B, cap] (or [.., cap, 1])."""
    q8 = _byte_view(q_fp8)
    kc = _byte_view(k_cache)
    _need(q8.dtype == torch.uint8 and q8.dim() == 4 and q8.shape[3] == DIM and q8.is_contiguous(),
          "q_fp8 must be contiguous [B, S, H, 128]")
    B, S, H = q8.shape[:3]
    _need(w_eff.dtype == torch.float32 and tuple(w_eff.shape) == (B, S, H) and w_eff.is_contiguous(), "bad w_eff")
    _need(kc.dtype == torch.uint8 and kc.dim() == 3 and kc.shape[2] == DIM and kc.stride(2) == 1
          and kc.stride(1) == DIM and kc.stride(0) % DIM == 0 and kc.shape[0] >= B, "bad k_cache")
    ks = k_scale.squeeze(-1) if k_scale.dim() == 3 else k_scale
    seq_stride = kc.stride(0) // DIM
    _need(ks.dtype == torch.float32 and ks.dim() == 2 and ks.shape[:2] == kc.shape[:2] and ks.stride(1) == 1
          and (ks.shape[0] == 1 or ks.stride(0) == seq_stride), "k_scale must share k_cache's sequence stride")
    _need(0 <= T <= kc.shape[1], "T exceeds the cache capacity")
    if scores is None:
        scores = torch.empty((B, S, T), dtype=torch.float32, device=q8.device)
    _need(scores.dtype == torch.float32 and tuple(scores.shape) == (B, S, T) and scores.is_contiguous(), "bad scores")
    rows = _rows(B, S, T, start_pos, seq_len, causal)
    st = _lib.load().lk_index_score(q8.data_ptr(), w_eff.data_ptr(), H, kc.data_ptr(), ks.data_ptr(),
                                    seq_stride, ctypes.byref(rows), scores.data_ptr(), _stream(q8))
    _lib.check("lk_index_score", st)
    return scores


def lk_decode_score(q: torch.Tensor, w: torch.Tensor, k_new: torch.Tensor, k_cache: torch.Tensor,
                    k_scale: torch.Tensor, T: int, start_pos: int = 0, seq_len: Optional[torch.Tensor] = None,
                    causal: bool = False, scores: Optional[torch.Tensor] = None,
                    q_fp8_out: Optional[torch.Tensor] = None, w_eff_out: Optional[torch.Tensor] = None,
                    rope=None) -> torch.Tensor:
    """One decode step up to the scores in one launch: writes k_new [B, 128] (bf16) to
    slot L-1 of each sequence's cache, quantizes q [B, 64, 128] (bf16) with weights
    w [B, 64] (float32), and returns masked scores [B, 1, T] (float32).  Optional
    q_fp8_out [B, 64, 128] and w_eff_out [B, 64] receive the quantized query; optional
    rope = (cos, sin) float32 [B, 32] rotates the query and the new key first."""
    _need(q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[-1] == DIM, "q must be contiguous bf16 [B, H, 128]")
    H = q.shape[-2]
    B = q.numel() // (H * DIM) if H > 0 else 0
    _need(w.dtype == torch.float32 and w.is_contiguous() and w.numel() == B * H, "w must be contiguous float32 [B, H]")
    _need(k_new.dtype == torch.bfloat16 and k_new.is_contiguous() and k_new.numel() == B * DIM,
          "k_new must be contiguous bf16 [B, 128]")
    kc = _byte_view(k_cache)
    _need(kc.dtype == torch.uint8 and kc.dim() == 3 and kc.shape[2] == DIM and kc.stride(2) == 1
          and kc.stride(1) == DIM and kc.stride(0) % DIM == 0 and kc.shape[0] >= B, "bad k_cache")
    ks = k_scale.squeeze(-1) if k_scale.dim() == 3 else k_scale
    seq_stride = kc.stride(0) // DIM
    _need(ks.dtype == torch.float32 and ks.dim() == 2 and ks.shape[:2] == kc.shape[:2] and ks.stride(1) == 1
          and (ks.shape[0] == 1 or ks.stride(0) == seq_stride), "k_scale must share k_cache's sequence stride")
    _need(0 <= T <= kc.shape[1], "T exceeds the cache capacity")
    if scores is None:
        scores = torch.empty((B, 1, T), dtype=torch.float32, device=q.device)
    _need(scores.dtype == torch.float32 and scores.numel() == B * T and scores.is_contiguous(), "bad scores")
    q8p = wep = None
    if q_fp8_out is not None or w_eff_out is not None:
        _need(q_fp8_out is not None and w_eff_out is not None, "pass both q_fp8_out and w_eff_out, or neither")
        q8o = _byte_view(q_fp8_out)
        _need(q8o.dtype == torch.uint8 and q8o.numel() == B * H * DIM and q8o.is_contiguous(), "bad q_fp8_out")
        _need(w_eff_out.dtype == torch.float32 and w_eff_out.numel() == B * H and w_eff_out.is_contiguous(),
              "bad w_eff_out")
        q8p, wep = q8o.data_ptr(), w_eff_out.data_ptr()
    rows = _rows(B, 1, T, start_pos, seq_len, causal)
    rc, rs = _rope_args(rope, B, q.device)
    st = _lib.load().lk_decode_score(q.data_ptr(), w.data_ptr(), H, k_new.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                     seq_stride, ctypes.byref(rows), scores.data_ptr(), q8p, wep, rc, rs, _stream(q))
    _lib.check("lk_decode_score", st)
    return scores


def lk_decode_select(q: torch.Tensor, w: torch.Tensor, k_new: torch.Tensor, k_cache: torch.Tensor,
                     k_scale: torch.Tensor, T: int, k: int, start_pos: int = 0,
                     seq_len: Optional[torch.Tensor] = None, causal: bool = False,
                     scores: Optional[torch.Tensor] = None, keep_scores: bool = True,
                     idx: Optional[torch.Tensor] = None, q_fp8_out: Optional[torch.Tensor] = None,
                     w_eff_out: Optional[torch.Tensor] = None, rope=None):
    """lk_decode_score and the per-row top-k from one call: returns (scores [B, 1, T] or
    None, idx [B, 1, k] int32).  Rows of at most LK_SELECT_FUSED_MAX_T (1024) keys run
    as one launch; with keep_scores=False (allowed only there) no score is written."""
    _need(q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[-1] == DIM, "q must be contiguous bf16 [B, H, 128]")
    H = q.shape[-2]
    B = q.numel() // (H * DIM) if H > 0 else 0
    _need(w.dtype == torch.float32 and w.is_contiguous() and w.numel() == B * H, "w must be contiguous float32 [B, H]")
    _need(k_new.dtype == torch.bfloat16 and k_new.is_contiguous() and k_new.numel() == B * DIM,
          "k_new must be contiguous bf16 [B, 128]")
    kc = _byte_view(k_cache)
    _need(kc.dtype == torch.uint8 and kc.dim() == 3 and kc.shape[2] == DIM and kc.stride(2) == 1
          and kc.stride(1) == DIM and kc.stride(0) % DIM == 0 and kc.shape[0] >= B, "bad k_cache")
    ks = k_scale.squeeze(-1) if k_scale.dim() == 3 else k_scale
    seq_stride = kc.stride(0) // DIM
    _need(ks.dtype == torch.float32 and ks.dim() == 2 and ks.shape[:2] == kc.shape[:2] and ks.stride(1) == 1
          and (ks.shape[0] == 1 or ks.stride(0) == seq_stride), "k_scale must share k_cache's sequence stride")
    _need(0 <= T <= kc.shape[1], "T exceeds the cache capacity")
    if keep_scores and scores is None:
        scores = torch.empty((B, 1, T), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores.dtype == torch.float32 and scores.numel() == B * T and scores.is_contiguous(), "bad scores")
    if idx is None:
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=q.device)
    _need(idx.dtype == torch.int32 and idx.numel() == B * k and idx.is_contiguous(), "bad idx")
    q8p = wep = None
    if q_fp8_out is not None or w_eff_out is not None:
        _need(q_fp8_out is not None and w_eff_out is not None, "pass both q_fp8_out and w_eff_out, or neither")
        q8o = _byte_view(q_fp8_out)
        _need(q8o.dtype == torch.uint8 and q8o.numel() == B * H * DIM and q8o.is_contiguous(), "bad q_fp8_out")
        _need(w_eff_out.dtype == torch.float32 and w_eff_out.numel() == B * H and w_eff_out.is_contiguous(),
              "bad w_eff_out")
        q8p, wep = q8o.data_ptr(), w_eff_out.data_ptr()
    rows = _rows(B, 1, T, start_pos, seq_len, causal)
    rc, rs = _rope_args(rope, B, q.device)
    st = _lib.load().lk_decode_select(q.data_ptr(), w.data_ptr(), H, k_new.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                      seq_stride, ctypes.byref(rows), scores.data_ptr() if scores is not None else None,
                                      q8p, wep, rc, rs, k, idx.data_ptr(), _stream(q))
    _lib.check("lk_decode_select", st)
    return scores, idx


def lk_topk(scores: torch.Tensor, k: int, start_pos: int = 0, seq_len: Optional[torch.Tensor] = None,
            causal: bool = False, idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indices [B, S, k] (int32) of the min(k, L) largest scores of each row's valid
    prefix [0, L); unused slots are -1."""
    _need(scores.dtype == torch.float32 and scores.dim() == 3 and scores.is_contiguous(),
          "scores must be contiguous float32 [B, S, T]")
    B, S, T = scores.shape
    if idx is None:
        idx = torch.empty((B, S, k), dtype=torch.int32, device=scores.device)
    _need(idx.dtype == torch.int32 and tuple(idx.shape) == (B, S, k) and idx.is_contiguous(), "bad idx")
    rows = _rows(B, S, T, start_pos, seq_len, causal)
    st = _lib.load().lk_topk(scores.data_ptr(), ctypes.byref(rows), k, idx.data_ptr(), _stream(scores))
    _lib.check("lk_topk", st)
    return idx


MLA_HEADS, MLA_LATENT, MLA_ROPE = 128, 512, 64


def lk_sparse_mla_decode(q_latent: torch.Tensor, q_rope: torch.Tensor, kv_latent: torch.Tensor,
                         kv_rope: torch.Tensor, idx: torch.Tensor, scale: float,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse MLA decode attention over selected slots: q_latent [B, 128, 512] and
    q_rope [B, 128, 64] (bf16), latent / rotary caches [>=B, cap, 512] / [>=B, cap, 64]
    (bf16, same sequence stride in rows), idx [B, n] int32 (-1 = unused) ->
    out [B, 128, 512] float32.  `workspace` (uint8, at least
    lk_sparse_mla_workspace_size bytes) is allocated when not given."""
    _need(q_latent.dtype == torch.bfloat16 and q_latent.is_contiguous() and q_latent.dim() == 3
          and tuple(q_latent.shape[1:]) == (MLA_HEADS, MLA_LATENT), "q_latent must be contiguous bf16 [B, 128, 512]")
    B = q_latent.shape[0]
    _need(q_rope.dtype == torch.bfloat16 and q_rope.is_contiguous() and tuple(q_rope.shape) == (B, MLA_HEADS, MLA_ROPE),
          "q_rope must be contiguous bf16 [B, 128, 64]")
    _need(kv_latent.dtype == torch.bfloat16 and kv_latent.dim() == 3 and kv_latent.shape[2] == MLA_LATENT
          and kv_latent.stride(2) == 1 and kv_latent.stride(1) == MLA_LATENT and kv_latent.shape[0] >= B,
          "kv_latent must be bf16 [>=B, cap, 512] with contiguous rows")
    stride = kv_latent.stride(0) // MLA_LATENT
    _need(kv_rope.dtype == torch.bfloat16 and kv_rope.dim() == 3 and kv_rope.shape[2] == MLA_ROPE
          and kv_rope.stride(2) == 1 and kv_rope.stride(1) == MLA_ROPE and kv_rope.shape[:2] == kv_latent.shape[:2]
          and (kv_rope.shape[0] == 1 or kv_rope.stride(0) // MLA_ROPE == stride),
          "kv_rope must be bf16 [.., cap, 64] sharing kv_latent's rows")
    _need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 2 and idx.shape[0] == B,
          "idx must be contiguous int32 [B, n]")
    n_idx = idx.shape[1]
    lib = _lib.load()
    need_ws = lib.lk_sparse_mla_workspace_size(B, n_idx)
    if workspace is None:
        workspace = torch.empty(max(need_ws, 16), dtype=torch.uint8, device=q_latent.device)
    _need(workspace.is_cuda and workspace.numel() * workspace.element_size() >= need_ws, "workspace too small")
    if out is None:
        out = torch.empty((B, MLA_HEADS, MLA_LATENT), dtype=torch.float32, device=q_latent.device)
    _need(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, MLA_HEADS, MLA_LATENT),
          "bad out")
    st = lib.lk_sparse_mla_decode(q_latent.data_ptr(), q_rope.data_ptr(), kv_latent.data_ptr(), kv_rope.data_ptr(),
                                  stride, kv_latent.shape[1], idx.data_ptr(), B, n_idx, float(scale), out.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(q_latent))
    _lib.check("lk_sparse_mla_decode", st)
    return out

