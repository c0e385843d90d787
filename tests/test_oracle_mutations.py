"""Planted mistakes in copies of the oracle must fail the pins (CPU only).

Each mutant is a plausible slip (a dropped term, a wrong causal offset, a
transposed or mis-sliced operand, a reversed tie rule); the matching pin from
the pin modules must reject it while accepting the real oracle.
"""
import numpy as np
import pytest

import oracle
from oracle.attention import _softmax_rows, visible_mask

import test_oracle_attention as A
import test_oracle_decode as DEC
import test_oracle_indexer as I
import test_oracle_sparse as S


def nonabs_no_rope(qn, qr, kn, kr, v, scale, causal=True, rows=None):
    return oracle.mla_nonabsorbed(qn, np.zeros_like(qr), kn, kr, v, scale, causal, rows)


def nonabs_top_left(qn, qr, kn, kr, v, scale, causal=True, rows=None):
    L, H, _ = qn.shape
    N = kn.shape[0]
    allowed = np.arange(N)[None, :] <= np.arange(L)[:, None]
    out = np.empty((L, H, v.shape[2]))
    for h in range(H):
        s = qn[:, h] @ kn[:, h].T + qr[:, h] @ kr.T
        out[:, h] = _softmax_rows(scale * s, allowed) @ v[:, h]
    return out


def nonabs_head0_keys(qn, qr, kn, kr, v, scale, causal=True, rows=None):
    return oracle.mla_nonabsorbed(qn, qr, np.broadcast_to(kn[:, :1], kn.shape).copy(), kr, v, scale, causal, rows)


def nonabs_unscaled_rope(qn, qr, kn, kr, v, scale, causal=True, rows=None):
    L, H, _ = qn.shape
    N = kn.shape[0]
    allowed = visible_mask(L, N, causal)
    out = np.empty((L, H, v.shape[2]))
    for h in range(H):
        s = scale * (qn[:, h] @ kn[:, h].T) + qr[:, h] @ kr.T
        out[:, h] = _softmax_rows(s, allowed) @ v[:, h]
    return out


def abs_value_tail(q, kv, scale, dv=512, causal=True, rows=None):
    """Takes the value from the last dv entries of the row instead of the first."""
    L, H, _ = q.shape
    N = kv.shape[0]
    allowed = visible_mask(L, N, causal)
    out = np.empty((L, H, dv))
    for h in range(H):
        out[:, h] = _softmax_rows(scale * (q[:, h] @ kv.T), allowed) @ kv[:, -dv:]
    return out


def sparse_minus_one_wraps(q, kv, idx, scale, dv=512, rows=None):
    idx = np.where(np.asarray(idx) < 0, kv.shape[0] - 1, idx)   # -1 read as the last row
    return oracle.mla_sparse_gather(q, kv, idx, scale, dv, rows)


def topk_high_index_ties(s, k):
    s = np.atleast_2d(s)
    out = np.full((s.shape[0], k), -1, dtype=np.int64)
    for r in range(s.shape[0]):
        n = s.shape[1]
        order = n - 1 - np.argsort(-s[r, ::-1], kind="stable")
        nv = int(np.isfinite(s[r]).sum())
        out[r, : min(k, nv)] = order[: min(k, nv)]
    return out


def topk_blocked_no_carry(s, k, block=3):
    s = np.atleast_2d(s)
    out = np.full((s.shape[0], k), -1, dtype=np.int64)
    for r in range(s.shape[0]):
        keep = np.zeros(0, dtype=np.int64)
        for b0 in range(0, s.shape[1], block):
            blk = np.arange(b0, min(s.shape[1], b0 + block))
            blk = blk[np.isfinite(s[r, blk])]
            order = np.lexsort((blk, -s[r, blk]))
            keep = np.concatenate([keep, blk[order]])[-k:] if len(blk) else keep   # forgets the order of the union
        out[r, : len(keep)] = keep
    return out


def scores_no_relu(q, k, w, causal=True, rows=None):
    L, N = q.shape[0], k.shape[0]
    s = np.einsum("ih,ihn->in", w, q @ k.T)
    if causal:
        s[np.arange(N)[None, :] > (N - L + np.arange(L))[:, None]] = -np.inf
    return s


def scores_relu_outside(q, k, w, causal=True, rows=None):
    s = scores_no_relu(q, k, w, causal)
    return np.where(np.isfinite(s), np.maximum(s, 0), s)


@pytest.mark.parametrize("mutant,pin", [
    (nonabs_no_rope, A.pin_nonabs_vs_sdpa),
    (nonabs_no_rope, A.pin_nonabs_golden),
    (nonabs_top_left, A.pin_nonabs_vs_sdpa),
    (nonabs_top_left, A.pin_nonabs_zero_query_prefix_mean),
    (nonabs_head0_keys, A.pin_nonabs_vs_sdpa),
    (nonabs_head0_keys, A.pin_nonabs_golden),
    (nonabs_unscaled_rope, A.pin_nonabs_vs_sdpa),
    (nonabs_unscaled_rope, A.pin_nonabs_rope_only),
])
def test_nonabsorbed_mutants_caught(mutant, pin, rng):
    args = (mutant,) if pin is A.pin_nonabs_golden else (mutant, rng)
    assert not pin(*args)


@pytest.mark.parametrize("pin", [A.pin_absorption_identity, A.pin_absorbed_vs_sdpa, A.pin_absorbed_brute])
def test_absorbed_value_slice_mutant_caught(pin, rng):
    assert not pin(abs_value_tail, rng)


def masked_no_causal(q, kv, idx, scale, dv=512, causal=True, rows=None):
    """Drops the causal term: selected keys past the query's limit get weight."""
    return oracle.mla_masked_dense(q, kv, idx, scale, dv, causal=False, rows=rows)


def sparse_dedup(q, kv, idx, scale, dv=512, rows=None):
    """Treats each index row as a set: a repeated index weighs once."""
    idx = np.asarray(idx)
    out = np.full(idx.shape, -1, dtype=np.int64)
    for r in range(idx.shape[0]):
        u = np.unique(idx[r][idx[r] >= 0])
        out[r, :len(u)] = u
    return oracle.mla_sparse_gather(q, kv, out, scale, dv, rows)


def test_masked_causal_mutant_caught(rng):
    assert not S.pin_masked_causal_clause(masked_no_causal, rng)


def test_gather_dedup_mutant_caught(rng):
    assert not S.pin_gather_repeats_per_occurrence(sparse_dedup, rng)


def test_sparse_minus_one_mutant_caught(rng):
    assert not S.pin_sparse_equals_masked_dense(sparse_minus_one_wraps, rng, pad=0.3)


def test_tie_rule_mutant_caught(rng):
    assert not I.pin_topk_subsets(topk_high_index_ties, rng)
    assert not I.pin_golden(oracle.indexer_scores, topk_high_index_ties)


def test_blocked_without_carry_mutant_caught(rng):
    assert not I.pin_topk_subsets(topk_blocked_no_carry, rng)


@pytest.mark.parametrize("mutant", [scores_no_relu, scores_relu_outside])
def test_score_mutants_caught(mutant, rng):
    assert not I.pin_golden(mutant, oracle.topk_full)
    assert not I.pin_fraction_brute(mutant, rng)


def paged_rows_swapped(kv_pages, page_table, seq_len):
    page_size = kv_pages.shape[1]
    n = np.arange(seq_len)
    return kv_pages[np.asarray(page_table)[n % page_size], n // page_size]


def paged_rows_by_slot(kv_pages, page_table, seq_len):
    n = np.arange(seq_len)                        # ignores the table: physical order
    return kv_pages.reshape(-1, kv_pages.shape[2])[n]


def decode_drops_newest_key(q, kv_pages, page_table, seq_lens, scale, dv=512):
    return oracle.mla_decode_paged(q, kv_pages, page_table, [max(0, int(n) - 1) for n in seq_lens], scale, dv)


@pytest.mark.parametrize("mutant", [paged_rows_swapped, paged_rows_by_slot])
def test_paged_rows_mutants_caught(mutant):
    assert not DEC.pin_paged_rows_hand(mutant)


def test_decode_mutant_caught(rng):
    assert not DEC.pin_decode_brute(decode_drops_newest_key, rng)


def test_real_oracle_passes_every_pin(rng):
    assert A.pin_nonabs_golden(oracle.mla_nonabsorbed)
    assert A.pin_nonabs_vs_sdpa(oracle.mla_nonabsorbed, rng)
    assert A.pin_nonabs_rope_only(oracle.mla_nonabsorbed, rng)
    assert A.pin_absorption_identity(oracle.mla_absorbed, rng)
    assert S.pin_sparse_equals_masked_dense(oracle.mla_sparse_gather, rng, pad=0.3)
    assert S.pin_masked_causal_clause(oracle.mla_masked_dense, rng)
    assert S.pin_gather_repeats_per_occurrence(oracle.mla_sparse_gather, rng)
    assert I.pin_topk_subsets(oracle.topk_full, rng)
    assert I.pin_golden(oracle.indexer_scores, oracle.topk_full)
    assert DEC.pin_paged_rows_hand(oracle.paged_rows)
    assert DEC.pin_decode_brute(oracle.mla_decode_paged, rng)
