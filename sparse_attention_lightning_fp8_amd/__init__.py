"""Lightning-indexer hot path for MI355X (gfx950): key write, fp8 index score with
mask, and per-row top-k, as hand-written HIP kernels behind a C ABI (include/lk.h).

The Python functions below only marshal torch tensors into that ABI.
"""
from ._lib import LkError, LkRows  # noqa: F401
from .api import (lk_decode_score, lk_decode_select, lk_index_score, lk_prepare, lk_quantize_keys,  # noqa: F401
                  lk_quantize_queries, lk_sparse_mla_decode, lk_topk)

__all__ = ["lk_quantize_keys", "lk_quantize_queries", "lk_prepare", "lk_index_score", "lk_decode_score", "lk_decode_select", "lk_topk", "lk_sparse_mla_decode", "LkError", "LkRows"]
