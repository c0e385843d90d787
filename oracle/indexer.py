"""Canonical indexer score and top-k selection in fp64 (test infrastructure only).

"Sparse prefill for GLM", section "Blocked top-k": the indexer picks the top-k
keys for every query from a score over 32 indexer heads; the blocked version
scores the keys a block at a time and folds every block into a running top-k
list, and picks the same keys as the full selection up to the order of equal
scores.

The pages do not print the score. The one used here is
    s[i, n] = sum_h w[i, h] * ReLU(q[i, h, :] . k[n, :])      for n <= p_i, else -inf
with p_i = N - L + i (queries at the last L positions). Reading for the
precision, which the pages leave open: the score is defined canonically as

    d[h] = (((0 + q_0 k_0) + q_1 k_1) + ... )   fp64, dims in ascending order
    s    = (((0 + w_0 max(d_0, 0)) + w_1 max(d_1, 0)) + ... )   fp64, heads in ascending order

with every product and sum rounded separately (no fused multiply-add). q and k
are bf16 values, so every product is exact in fp64, and whenever the exponent
spread of a (query head, key) pair allows it every partial sum is exact as well;
then any summation order (BLAS included) gives the same d. `exact_dot_flags`
finds the pairs where that guarantee fails, and only those are summed in the
sequential order above.

Ties are broken by the lower key index (so the top-k set is unique); a row with
fewer than k visible keys returns all of them followed by -1.
"""
from __future__ import annotations

import math

import numpy as np


def _exp_stats(x: np.ndarray):
    """Per-row (max exponent, lowest possible significant-bit exponent) of bf16-valued data.

    For a nonzero bf16 value x = m * 2^e (0.5 <= |m| < 1), |x| < 2^e and x is a
    multiple of 2^(e - 8). Rows of zeros get (-inf-like, +inf-like) sentinels.
    """
    m, e = np.frexp(x)
    nz = x != 0
    emax = np.where(nz, e, -100000).max(axis=-1)
    elsb = np.where(nz, e - 8, 100000).min(axis=-1)
    return emax, elsb


def _span(x: np.ndarray) -> np.ndarray:
    e, l = _exp_stats(x)
    return np.where(e > -100000, e - l, -10**6)


def exact_dot_flags(q_rows: np.ndarray, k: np.ndarray, span_k=None) -> np.ndarray:
    """[Hi, N] bool: True where the fp64 dot q_h . k_n is NOT guaranteed exact in every order.

    All partial sums are integer multiples of 2^(lq + lk) and bounded by
    Di * 2^(eq + ek); they are exact in fp64 if Di * 2^(eq+ek) <= 2^(53+lq+lk).
    """
    Di = q_rows.shape[-1]
    lg = math.ceil(math.log2(Di))
    if span_k is None:
        span_k = _span(k)
    return (_span(q_rows)[:, None] + span_k[None, :]) > (53 - lg)


def _head_dots(qi: np.ndarray, k: np.ndarray, span_k=None) -> np.ndarray:
    """d[h, n] for one query, [Hi, Di] x [N, Di] -> [Hi, N], canonical fp64 values."""
    d = qi @ k.T
    flags = exact_dot_flags(qi, k, span_k)
    if flags.any():
        hs, ns = np.nonzero(flags)
        acc = np.zeros(len(hs))
        for c in range(qi.shape[1]):
            acc = acc + qi[hs, c] * k[ns, c]
        d[hs, ns] = acc
    return d


def indexer_scores(q, k, w, causal=True, rows=None):
    """Canonical scores s [len(rows), N] (float64, -inf where not visible).

    q [L,Hi,Di] and k [N,Di] hold bf16 values as float64, w [L,Hi] fp32 values as float64.
    """
    L, Hi, _ = q.shape
    N = k.shape[0]
    if causal and L > N:
        raise ValueError("causal indexer needs L <= N")
    rows = np.arange(L) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), N))
    span_k = _span(k)
    for r, i in enumerate(rows):
        d = _head_dots(q[i], k, span_k)
        s = np.zeros(N)
        for h in range(Hi):
            s = s + w[i, h] * np.maximum(d[h], 0.0)
        if causal:
            s[N - L + i + 1:] = -np.inf
        out[r] = s
    return out


def topk_full(s: np.ndarray, k: int) -> np.ndarray:
    """Full top-k by (score descending, index ascending) over each row; -1 pads.

    The definition written out: a stable sort of the negated scores keeps equal
    scores in ascending index order; the first k visible entries are the set.
    """
    s = np.atleast_2d(s)
    out = np.full((s.shape[0], k), -1, dtype=np.int64)
    for r in range(s.shape[0]):
        order = np.argsort(-s[r], kind="stable")
        nvis = int(np.isfinite(s[r]).sum())
        take = order[: min(k, nvis)]
        out[r, : len(take)] = take
    return out


def topk_blocked(s: np.ndarray, k: int, block: int) -> np.ndarray:
    """Running top-k over blocks of `block` keys ("Sparse prefill for GLM", "Blocked top-k").

    Start from an empty list; for each block, take the top k of (list + block)
    by (score descending, index ascending). A final partial block is allowed.
    """
    s = np.atleast_2d(s)
    N = s.shape[1]
    out = np.full((s.shape[0], k), -1, dtype=np.int64)
    for r in range(s.shape[0]):
        keep = np.zeros(0, dtype=np.int64)
        for b0 in range(0, N, block):
            blk = np.arange(b0, min(N, b0 + block))
            blk = blk[np.isfinite(s[r, blk])]
            cand = np.concatenate([keep, blk])
            order = np.lexsort((cand, -s[r, cand]))
            keep = cand[order[:k]]
        out[r, : len(keep)] = keep
    return out
