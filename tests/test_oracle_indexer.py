"""Pins for the indexer score and top-k oracle (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import bf16_bits, bf16_to_f32, gen_indexer, gen_indexer_exact, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return bf16_to_f32(bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def pin_golden(score_fn, topk_fn):
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    q, k, w = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "w"))
    s = score_fn(q, k, w)
    exp = np.array([[float(x) for x in r] for r in g["scores"]])
    if not np.array_equal(s, exp):
        return False
    for kk, sets in g["topk"].items():
        got = topk_fn(s, int(kk))
        if [sorted(r.tolist()) for r in got] != [sorted(r) for r in sets]:
            return False
    return True


def pin_fraction_brute(score_fn, rng, w_shift=0.0):
    """Exact rational scores (Fractions) vs the fp64 canonical score on tiny random bf16
    inputs; w_shift > 0 draws weights of either sign."""
    L, N, H, D = 3, 12, 4, 8
    q = _bf16(rng.standard_normal((L, H, D)))
    k = _bf16(rng.standard_normal((N, D)))
    w = (rng.random((L, H)) - w_shift).astype(np.float32).astype(np.float64)
    s = score_fn(q, k, w)
    for i in range(L):
        for n in range(N):
            if n > N - L + i:
                if s[i, n] != -np.inf:
                    return False
                continue
            ex = brute.indexer_score_exact(q[i].tolist(), k[n].tolist(), w[i].tolist())
            # canonical value = exact products/dots, then H roundings in the head sum
            if abs(Fraction(s[i, n]) - ex) > Fraction(2 * H) * Fraction(2) ** -53 * (abs(ex) + 1):
                return False
    return True


def pin_exact_inputs(score_fn):
    """On exact-arithmetic inputs the canonical score equals the rational score exactly."""
    g = gen_indexer_exact(77, 3, 20, Hi=6, Di=16)
    q, k, w = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    s = score_fn(q, k, w)
    for i in range(3):
        for n in range(20 - 3 + i + 1):
            if Fraction(s[i, n]) != brute.indexer_score_exact(q[i].tolist(), k[n].tolist(), w[i].tolist()):
                return False
    return True


def pin_topk_subsets(topk_fn, rng, lo=0):
    for trial in range(20):
        N = int(rng.integers(1, 9))
        k = int(rng.integers(1, 6))
        s = rng.integers(lo, 4, size=N).astype(np.float64)       # many ties
        s[rng.random(N) < 0.2] = -np.inf                          # invisible keys
        got = set(int(x) for x in topk_fn(s[None], k)[0] if x >= 0)
        ref = brute.topk_by_subsets([None if not np.isfinite(x) else x for x in s], k)
        if got != ref:
            return False
    return True


def test_golden_hand_example():
    assert pin_golden(oracle.indexer_scores, oracle.topk_full)


def test_golden_hand_example_blocked():
    for b in (1, 2, 4, 6):
        assert pin_golden(oracle.indexer_scores, lambda s, k, b=b: oracle.topk_blocked(s, k, b))


def test_scores_vs_exact_fractions(rng):
    assert pin_fraction_brute(oracle.indexer_scores, rng)


def test_scores_vs_exact_fractions_signed_weights(rng):
    assert pin_fraction_brute(oracle.indexer_scores, rng, w_shift=0.5)


def test_exact_inputs_are_exact():
    assert pin_exact_inputs(oracle.indexer_scores)


def test_topk_brute_force_subsets(rng):
    assert pin_topk_subsets(oracle.topk_full, rng)


def test_topk_brute_force_subsets_negative_scores(rng):
    assert pin_topk_subsets(oracle.topk_full, rng, lo=-3)


def test_topk_blocked_brute_force_subsets(rng):
    for b in (1, 3):
        assert pin_topk_subsets(lambda s, k, b=b: oracle.topk_blocked(s, k, b), rng)


def test_zero_query_selects_lowest_indices():
    g = gen_indexer(5, 4, 64, Hi=4, Di=16)
    q, k, w = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    s = oracle.indexer_scores(np.zeros_like(q), k, w)
    assert np.all(s[np.isfinite(s)] == 0)
    got = oracle.topk_full(s, 10)
    assert all(sorted(r) == list(range(10)) for r in got.tolist())


def test_constant_and_increasing_scores():
    s = np.zeros((1, 50))
    assert sorted(oracle.topk_full(s, 7)[0].tolist()) == list(range(7))
    s = np.arange(50, dtype=np.float64)[None]
    assert sorted(oracle.topk_full(s, 7)[0].tolist()) == list(range(43, 50))


def test_one_hot_weight_is_plain_relu_dot():
    g = gen_indexer(6, 3, 40, Hi=5, Di=16)
    q, k = to_f64(g["q_idx"]), to_f64(g["k_idx"])
    w = np.zeros((3, 5))
    w[:, 2] = 1.0
    s = oracle.indexer_scores(q, k, w, causal=False)
    for i in range(3):
        ref = np.array([max(float(sum(Fraction(a) * Fraction(b) for a, b in zip(q[i, 2], k[n]))), 0.0) for n in range(40)])
        assert np.array_equal(s[i], ref)


def test_power_of_two_weight_scaling():
    g = gen_indexer(7, 4, 80, Hi=6, Di=16)
    q, k, w = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    s1 = oracle.indexer_scores(q, k, w)
    s2 = oracle.indexer_scores(q, k, w * 8.0)
    assert np.array_equal(s2, s1 * 8.0)
    assert np.array_equal(oracle.topk_full(s1, 9), oracle.topk_full(s2, 9))


@pytest.mark.parametrize("block", [1, 3, 7, 4096, 200])
def test_blocked_equals_full(block):
    g = gen_indexer_exact(9, 6, 200, Hi=4, Di=16)     # exact ties
    s = oracle.indexer_scores(to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"]))
    for k in (1, 5, 40, 195, 250):
        assert np.array_equal(np.sort(oracle.topk_full(s, k), axis=1), np.sort(oracle.topk_blocked(s, k, block), axis=1))


def test_fewer_visible_than_k_pads():
    g = gen_indexer(10, 4, 6, Hi=2, Di=8)
    s = oracle.indexer_scores(to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"]))
    got = oracle.topk_full(s, 5)
    assert sorted(got[0].tolist()) == [-1, -1, 0, 1, 2]       # query 0 at position 2 sees 3 keys
    assert got[3].min() >= 0 and len(set(got[3].tolist())) == 5   # query 3 at position 5 sees 6 keys


def test_exponent_spread_uses_sequential_sum():
    """A pair whose fp64 dot is not exact in every order is summed in ascending dim order."""
    q = np.zeros((1, 1, 4))
    q[0, 0] = [2.0 ** 60, 1.0, -(2.0 ** 60), 1.0]
    k = np.ones((1, 4))
    flags = oracle.exact_dot_flags(q[0], k)
    assert flags[0, 0]
    s = oracle.indexer_scores(q, k, np.ones((1, 1)))
    seq = 0.0
    for c in range(4):
        seq = seq + q[0, 0, c] * k[0, c]
    assert s[0, 0] == max(seq, 0.0) and seq == 1.0        # ((2^60 + 1) - 2^60) + 1 = 0 + 1
    g = gen_indexer(11, 2, 30)
    assert not oracle.exact_dot_flags(to_f64(g["q_idx"])[0], to_f64(g["k_idx"])).all()
