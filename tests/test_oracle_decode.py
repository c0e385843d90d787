"""Pins of the paged decode oracle (CPU): page lookup by hand, brute force, closed
forms and invariants that do not go through the oracle's own formula."""
import numpy as np

import oracle
from oracle import brute


def pin_paged_rows_hand(rows_fn):
    # 4 physical pages of 2 rows; the sequence lives in pages 3, 0, 2 (in that order)
    pages = np.arange(4 * 2 * 3, dtype=np.float64).reshape(4, 2, 3)
    try:
        rows = rows_fn(pages, [3, 0, 2, 1], 5)
    except IndexError:                        # a walk that leaves the pages is wrong too
        return False
    expect = np.array([pages[3, 0], pages[3, 1], pages[0, 0], pages[0, 1], pages[2, 0]])
    return rows.shape == expect.shape and np.array_equal(rows, expect)


def pin_decode_brute(decode_fn, rng):
    B, H, D, dv, ps, P = 2, 2, 5, 3, 2, 6
    pages = rng.standard_normal((P, ps, D))
    table = np.array([[4, 1, 5], [2, 0, 3]])
    lens = [5, 3]
    q = rng.standard_normal((B, H, D))
    got = decode_fn(q, pages, table, lens, 0.7, dv=dv)
    for b in range(B):
        kv = []
        for n in range(lens[b]):                      # the page walk written out by hand
            kv.append(list(pages[table[b][n // ps]][n % ps]))
        ref = brute.absorbed([[list(q[b, h]) for h in range(H)]], kv, 0.7, dv)
        for h in range(H):
            if not np.allclose(got[b, h], ref[0][h], rtol=0, atol=1e-13):
                return False
    return True


def test_paged_rows_hand_built_table():
    assert pin_paged_rows_hand(oracle.paged_rows)


def test_decode_matches_brute_force():
    assert pin_decode_brute(oracle.mla_decode_paged, np.random.default_rng(7))


def test_decode_closed_forms():
    rng = np.random.default_rng(8)
    pages = rng.standard_normal((3, 4, 6))
    q = rng.standard_normal((3, 2, 6))
    table = np.array([[2, 0, 1], [1, 2, 0], [0, 1, 2]])
    out = oracle.mla_decode_paged(q, pages, table, [0, 1, 12], 0.5, dv=4)
    assert np.all(out[0] == 0)                                    # empty sequence
    assert np.array_equal(out[1], np.tile(pages[1, 0, :4], (2, 1)))   # one key: its value row
    q0 = np.zeros_like(q)
    out0 = oracle.mla_decode_paged(q0, pages, table, [0, 1, 12], 0.5, dv=4)
    seq = np.concatenate([pages[0], pages[1], pages[2]])
    assert np.allclose(out0[2], np.tile(seq[:, :4].mean(0), (2, 1)), atol=1e-14)   # zero query: mean


def test_decode_invariant_to_page_placement_and_equals_contiguous():
    rng = np.random.default_rng(9)
    P, ps, D = 8, 4, 7
    pages = rng.standard_normal((P, ps, D))
    q = rng.standard_normal((1, 3, D))
    table = np.array([[5, 2, 7, 0]])
    base = oracle.mla_decode_paged(q, pages, table, [14], 0.3, dv=5)
    perm = rng.permutation(P)                     # move every page to a new slot
    moved = np.empty_like(pages)
    moved[perm] = pages
    base2 = oracle.mla_decode_paged(q, moved, perm[table], [14], 0.3, dv=5)
    assert np.array_equal(base, base2)
    contiguous = np.concatenate([pages[5], pages[2], pages[7], pages[0]])[:14]
    ref = oracle.mla_absorbed(q[0][None], contiguous, 0.3, dv=5)[0]
    assert np.allclose(base[0], ref, atol=1e-14)
