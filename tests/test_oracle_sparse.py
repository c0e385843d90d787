"""Pins for the sparse (gather) and masked-dense oracles and the gate (CPU only).

Maps the named tests of "Sparse prefill for GLM", section "Accuracy and tests":
sparse output matches dense under the mask, short and gated contexts take the
dense path unchanged, query blocks match.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from synth import gen_topk_indices


def _abs_inputs(rng, L, N, H=3, D=10):
    return rng.standard_normal((L, H, D)), rng.standard_normal((N, D))


def pin_sparse_equals_masked_dense(fn_sparse, rng, L=6, N=40, topk=9, pad=0.2):
    q, kv = _abs_inputs(rng, L, N)
    idx = gen_topk_indices(int(rng.integers(1 << 30)), L, N, topk, pad_frac=pad)
    a = fn_sparse(q, kv, idx, 0.3, dv=7)
    b = oracle.mla_masked_dense(q, kv, idx, 0.3, dv=7)
    return np.allclose(a, b, rtol=0, atol=1e-12)


def pin_sparse_brute(fn_sparse, rng):
    L, N, topk = 3, 8, 4
    q, kv = _abs_inputs(rng, L, N, H=2, D=4)
    idx = gen_topk_indices(5, L, N, topk)
    sel = [set(int(x) for x in r if x >= 0) for r in idx]
    ref = np.array(brute.absorbed(q.tolist(), kv.tolist(), 0.7, 3, sel=sel))
    return np.allclose(fn_sparse(q, kv, idx, 0.7, dv=3), ref, rtol=0, atol=1e-12)


def pin_masked_causal_clause(fn_masked, rng):
    """Selected keys past a query's causal limit stay masked ("Sparse prefill for GLM",
    section "The dense mask": the selection mask is combined with the causal mask).

    Queries sit at positions 5..8 of N = 9; every row selects keys past its limit.
    Reference: the pure-Python brute force over the explicit set of keys that are
    both selected and visible, and the closed form of query 0, whose only selected
    visible key is key 0, so its output is that key's value row exactly.
    """
    L, N, H, D, dv = 4, 9, 2, 5, 3
    q, kv = rng.standard_normal((L, H, D)), rng.standard_normal((N, D))
    idx = np.array([[0, 7, 8, -1], [2, 6, 8, 3], [1, 8, 4, 7], [0, 1, 2, 8]])
    sel = [{int(x) for x in r if 0 <= x <= N - L + i} for i, r in enumerate(idx)]
    assert sel[0] == {0} and sel[1] == {2, 3, 6} and sel[2] == {1, 4, 7}   # the limit cuts every row but the last
    got = fn_masked(q, kv, idx, 0.5, dv=dv)
    ref = np.array(brute.absorbed(q.tolist(), kv.tolist(), 0.5, dv, sel=sel))
    first = np.broadcast_to(kv[0, :dv], (H, dv))
    return bool(np.allclose(got, ref, rtol=0, atol=1e-12) and np.array_equal(got[0], first))


def pin_gather_repeats_per_occurrence(fn_sparse, rng):
    """A repeated index weighs once per occurrence in the gather form ("Sparse prefill
    for GLM", section "Sparse attention": the chosen rows are gathered, so a key listed
    twice is two rows of the gathered block).

    Closed form: with a zero query every copy has score 0, so the output is the plain
    mean over the copies: a key listed twice and one listed once give (2 v_a + v_b) / 3
    (a set would give (v_a + v_b) / 2). Brute force: the explicitly gathered list of
    copies for random queries.
    """
    L, N, H, D, dv = 3, 8, 2, 6, 4
    q, kv = rng.standard_normal((L, H, D)), rng.standard_normal((N, D))
    q[0] = 0.0
    idx = np.array([[3, 5, 3, -1], [1, 1, 1, 6], [2, 7, 7, 0]])
    got = fn_sparse(q, kv, idx, 0.4, dv=dv)
    closed = np.broadcast_to((2 * kv[3, :dv] + kv[5, :dv]) / 3, (H, dv))
    ref = np.array([brute.gathered(q[i].tolist(), kv.tolist(), idx[i].tolist(), 0.4, dv) for i in range(L)])
    return bool(np.allclose(got[0], closed, rtol=0, atol=1e-14) and np.allclose(got, ref, rtol=0, atol=1e-12))


def test_masked_dense_causal_clause(rng):
    assert pin_masked_causal_clause(oracle.mla_masked_dense, rng)


def test_gather_repeats_count_per_occurrence(rng):
    assert pin_gather_repeats_per_occurrence(oracle.mla_sparse_gather, rng)


def test_sparse_matches_dense_under_mask(rng):
    assert pin_sparse_equals_masked_dense(oracle.mla_sparse_gather, rng)


def test_sparse_brute_force(rng):
    assert pin_sparse_brute(oracle.mla_sparse_gather, rng)


def test_sparse_short_context_is_dense(rng):
    """topk >= visible keys: every visible key is selected, so sparse == plain dense attention."""
    L, N = 5, 12
    q, kv = _abs_inputs(rng, L, N)
    idx = gen_topk_indices(3, L, N, topk=N)
    a = oracle.mla_sparse_gather(q, kv, idx, 0.3, dv=6)
    b = oracle.mla_absorbed(q, kv, 0.3, dv=6)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_sparse_permutation_invariant(rng):
    L, N = 4, 30
    q, kv = _abs_inputs(rng, L, N)
    idx = gen_topk_indices(11, L, N, 8, pad_frac=0.25)
    perm = np.stack([rng.permutation(r) for r in idx])
    a = oracle.mla_sparse_gather(q, kv, idx, 0.3, dv=6)
    b = oracle.mla_sparse_gather(q, kv, perm, 0.3, dv=6)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_sparse_query_blocks_match(rng):
    """Query blocks ("Sparse attention": chunks longer than the block split into blocks) change nothing."""
    L, N = 9, 30
    q, kv = _abs_inputs(rng, L, N)
    idx = gen_topk_indices(12, L, N, 6)
    full = oracle.mla_sparse_gather(q, kv, idx, 0.3, dv=6)
    blocks = np.concatenate([oracle.mla_sparse_gather(q, kv, idx, 0.3, dv=6, rows=range(b, min(L, b + 4)))
                             for b in range(0, L, 4)])
    assert np.array_equal(full, blocks)


def test_sparse_empty_row_is_zero(rng):
    L, N = 3, 10
    q, kv = _abs_inputs(rng, L, N)
    idx = np.full((L, 4), -1, dtype=np.int32)
    idx[1] = [0, 3, -1, 5]
    out = oracle.mla_sparse_gather(q, kv, idx, 0.3, dv=6)
    assert np.all(out[0] == 0) and np.all(out[2] == 0) and np.any(out[1] != 0)
    assert np.allclose(out, oracle.mla_masked_dense(q, kv, idx, 0.3, dv=6, causal=False), atol=1e-13)


@pytest.mark.parametrize("flag,B,L,N,expect", [
    (True, 1, 512, 16384, True),
    (True, 1, 512, 16383, False),     # below the minimum context
    (True, 2, 512, 131072, False),    # batches keep the masked dense path
    (True, 1, 1, 131072, False),      # decode (one query) is untouched
    (False, 1, 512, 131072, False),   # switched off in the config
    (True, 1, 2, 16384, True),
])
def test_gate_truth_table(flag, B, L, N, expect):
    assert oracle.use_sparse(flag, B, L, N) is expect


def test_gate_min_context_override():
    assert oracle.use_sparse(True, 1, 4, 100, min_context=100)
    assert not oracle.use_sparse(True, 1, 4, 99, min_context=100)


def test_gated_prefill_uses_masked_dense(rng):
    """Below the minimum context the composed prefill is exactly the masked dense path."""
    L, N, topk = 4, 24, 6
    q, kv = _abs_inputs(rng, L, N, H=2, D=8)
    q_idx = rng.standard_normal((L, 2, 4)).astype(np.float32).astype(np.float64)
    k_idx = rng.standard_normal((N, 4)).astype(np.float32).astype(np.float64)
    w = rng.random((L, 2))
    out_g, idx = oracle.dsa_prefill(q, kv, q_idx, k_idx, w, topk, 0.3, dv=5, min_context=1000)
    assert np.array_equal(out_g, oracle.mla_masked_dense(q, kv, idx, 0.3, dv=5))
    out_s, idx2 = oracle.dsa_prefill(q, kv, q_idx, k_idx, w, topk, 0.3, dv=5, min_context=N)
    assert np.array_equal(idx, idx2)
    assert np.allclose(out_s, out_g, rtol=0, atol=1e-12)
