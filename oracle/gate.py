"""Dense/sparse gate and the composed DSA prefill (test infrastructure only).

"Sparse prefill for GLM", section "When it runs": the sparse path runs only when
it is switched on, the batch holds one sequence, the call is a prefill chunk
(more than one query) and the cache holds at least the minimum context
(16384 positions by default); otherwise the masked dense path runs.
"""
from __future__ import annotations

from .attention import mla_masked_dense, mla_sparse_gather
from .indexer import indexer_scores, topk_full

SPARSE_PREFILL_DEFAULT = True
SPARSE_PREFILL_MIN_CONTEXT_DEFAULT = 16384


def use_sparse(sparse_prefill: bool, B: int, L: int, N: int,
               min_context: int = SPARSE_PREFILL_MIN_CONTEXT_DEFAULT) -> bool:
    """The gate predicate; N is the number of cached positions including this chunk."""
    return bool(sparse_prefill) and B == 1 and L > 1 and N >= min_context


def dsa_prefill(q, kv, q_idx, k_idx, w, topk, scale, dv=512, B=1,
                sparse_prefill=SPARSE_PREFILL_DEFAULT,
                min_context=SPARSE_PREFILL_MIN_CONTEXT_DEFAULT, rows=None):
    """One chunk of DSA prefill for one sequence: indexer top-k, then the gated attention."""
    L = q.shape[0]
    N = kv.shape[0]
    import numpy as np
    rows = np.arange(L) if rows is None else np.asarray(rows)
    idx = np.full((L, topk), -1, dtype=np.int64)
    idx[rows] = topk_full(indexer_scores(q_idx, k_idx, w, rows=rows), topk)
    if use_sparse(sparse_prefill, B, L, N, min_context):
        return mla_sparse_gather(q, kv, idx, scale, dv, rows=rows), idx
    return mla_masked_dense(q, kv, idx, scale, dv, rows=rows), idx
