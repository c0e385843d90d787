"""Naive fp64 softmax attention for MLA prefill (test infrastructure only).

Causal convention (bottom-right): the L queries are the last L positions of an
N-position context, so query i sits at position p_i = N - L + i and key n is
visible to it iff n <= p_i. For L = N this is the ordinary j <= i rule.

Softmax over a row with no visible / selected key is undefined; this oracle
(and the library) return zeros for such a row.
"""
from __future__ import annotations

import numpy as np


def visible_mask(L: int, N: int, causal: bool = True, rows=None) -> np.ndarray:
    """[len(rows), N] bool: key n visible to query i (bottom-right causal)."""
    if causal and L > N:
        raise ValueError("causal attention needs L <= N")
    rows = np.arange(L) if rows is None else np.asarray(rows)
    if not causal:
        return np.ones((len(rows), N), dtype=bool)
    pos = N - L + rows
    return np.arange(N)[None, :] <= pos[:, None]


def _softmax_rows(s: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Row softmax of s restricted to allowed entries (others get weight 0)."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(s - m), 0.0)
    z = e.sum(axis=-1, keepdims=True)
    return np.divide(e, z, out=np.zeros_like(e), where=z > 0)


def mla_nonabsorbed(qn, qr, kn, kr, v, scale, causal=True, rows=None):
    """Non-absorbed MLA prefill.

    Fornax part 5, "What the kernel has to compute": the score is the sum of a
    contraction over the non-rope dims (per head) and a contraction over the
    rope dims against a rope key that is shared by all heads; the output is
    softmax(score) times the per-head value.

    qn [L,H,Dn], qr [L,H,Dr], kn [N,H,Dn], kr [N,Dr], v [N,H,Dv] (float64).
    Returns out [len(rows),H,Dv].
    """
    L, H, _ = qn.shape
    N = kn.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    allowed = visible_mask(L, N, causal, rows)
    out = np.empty((len(rows), H, v.shape[2]))
    for h in range(H):
        s = qn[rows, h, :] @ kn[:, h, :].T + qr[rows, h, :] @ kr.T
        p = _softmax_rows(scale * s, allowed)
        out[:, h, :] = p @ v[:, h, :]
    return out


def mla_absorbed(q, kv, scale, dv=512, causal=True, rows=None):
    """Absorbed (latent-space) dense MLA prefill.

    "Sparse prefill for GLM", section "Sparse attention": every position has one
    joined latent+rope row that all heads share; the score is the contraction of
    the latent-space query with that row and the value is its latent part
    (the first dv entries).

    q [L,H,D], kv [N,D] (float64). Returns out [len(rows),H,dv].
    """
    L, H, _ = q.shape
    N = kv.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    allowed = visible_mask(L, N, causal, rows)
    out = np.empty((len(rows), H, dv))
    vals = kv[:, :dv]
    for h in range(H):
        p = _softmax_rows(scale * (q[rows, h, :] @ kv.T), allowed)
        out[:, h, :] = p @ vals
    return out


def _selection_mask(idx: np.ndarray, N: int) -> np.ndarray:
    """[rows, N] bool from an index list; entries outside [0, N) (e.g. -1) are ignored."""
    m = np.zeros((idx.shape[0], N), dtype=bool)
    r, c = np.nonzero((idx >= 0) & (idx < N))
    m[r, idx[r, c]] = True
    return m


def mla_masked_dense(q, kv, idx, scale, dv=512, causal=True, rows=None):
    """Dense absorbed attention under a top-k boolean mask (the pre-sparse path).

    "Sparse prefill for GLM", section "The dense mask": the indexer's choice is
    turned into a boolean mask with one row per query and one column per key,
    and attention runs over every key with the others masked out.

    idx [L,topk] int (-1 = empty slot). Returns out [len(rows),H,dv].
    """
    L, H, _ = q.shape
    N = kv.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    allowed = visible_mask(L, N, causal, rows) & _selection_mask(np.asarray(idx)[rows], N)
    out = np.empty((len(rows), H, dv))
    vals = kv[:, :dv]
    for h in range(H):
        p = _softmax_rows(scale * (q[rows, h, :] @ kv.T), allowed)
        out[:, h, :] = p @ vals
    return out


def mla_sparse_gather(q, kv, idx, scale, dv=512, rows=None):
    """Sparse absorbed attention over gathered rows.

    "Sparse prefill for GLM", section "Sparse attention": for each query only the
    rows it picked are gathered from the joined cache; all heads share that
    gathered block, and softmax runs over it alone. Entries equal to -1 (or
    otherwise outside [0, N)) are skipped. A repeated index counts once per
    occurrence, as in a gather.

    Returns out [len(rows),H,dv].
    """
    L, H, _ = q.shape
    N = kv.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), H, dv))
    for r, i in enumerate(rows):
        sel = np.asarray(idx[i])
        sel = sel[(sel >= 0) & (sel < N)]
        if len(sel) == 0:
            continue
        g = kv[sel]                              # gathered block [t, D], shared by all heads
        s = scale * (q[i] @ g.T)                 # [H, t]
        p = _softmax_rows(s, np.ones_like(s, dtype=bool))
        out[r] = p @ g[:, :dv]
    return out


def paged_rows(kv_pages, page_table, seq_len):
    """The contiguous cache of one sequence rebuilt from a paged one: row n of the
    sequence is row n % page_size of page page_table[n // page_size] ("Apple M3 vs M5
    kernels", section "Paged KV: alignment follows the tile": every row is addressed
    on its own through the page pointers, so no tile has to sit inside one page).

    kv_pages [P,page_size,D], page_table [max_pages] int, seq_len int -> [seq_len,D].
    """
    page_size = kv_pages.shape[1]
    n = np.arange(seq_len)
    return kv_pages[np.asarray(page_table)[n // page_size], n % page_size]


def mla_decode_paged(q, kv_pages, page_table, seq_lens, scale, dv=512):
    """One decode step of absorbed MLA over a paged joined cache.

    "Sparse prefill for GLM", section "When it runs": decode (one new query per
    sequence) keeps the dense absorbed path; the new token's key is already in the
    cache, so the query sits at the last of seq_len positions and sees all of them.

    q [B,H,576], kv_pages [P,page_size,576], page_table [B,max_pages], seq_lens [B].
    A sequence of length 0 gets zeros. Returns out [B,H,dv].
    """
    B, H, _ = q.shape
    out = np.zeros((B, H, dv))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        kv = paged_rows(kv_pages, page_table[b], n)
        out[b] = mla_absorbed(q[b][None], kv, scale, dv)[0]
    return out
