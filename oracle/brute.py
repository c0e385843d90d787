"""Pure-Python brute force for tiny inputs (test infrastructure only).

Independent of the NumPy oracle: scalar loops, ``math.fsum`` and
``fractions.Fraction``; used only to pin the NumPy oracle on tiny shapes.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction


def attention_rows(scores, values, allowed):
    """softmax over allowed entries of each score row, times values (lists of floats)."""
    out = []
    for srow, arow in zip(scores, allowed):
        idx = [j for j, a in enumerate(arow) if a]
        if not idx:
            out.append([0.0] * len(values[0]))
            continue
        m = max(srow[j] for j in idx)
        e = {j: math.exp(srow[j] - m) for j in idx}
        z = math.fsum(e.values())
        out.append([math.fsum(e[j] * values[j][c] for j in idx) / z for c in range(len(values[0]))])
    return out


def nonabsorbed(qn, qr, kn, kr, v, scale):
    """Causal (bottom-right) non-absorbed MLA with Python scalars; nested lists in, nested lists out."""
    L, H, N = len(qn), len(qn[0]), len(kn)
    out = [[None] * H for _ in range(L)]
    for h in range(H):
        scores, allowed = [], []
        for i in range(L):
            row = []
            for j in range(N):
                nope = math.fsum(qn[i][h][c] * kn[j][h][c] for c in range(len(qn[i][h])))
                rope = math.fsum(qr[i][h][c] * kr[j][c] for c in range(len(qr[i][h])))
                row.append(scale * (nope + rope))
            scores.append(row)
            allowed.append([j <= N - L + i for j in range(N)])
        vals = [v[j][h] for j in range(N)]
        res = attention_rows(scores, vals, allowed)
        for i in range(L):
            out[i][h] = res[i]
    return out


def absorbed(q, kv, scale, dv, sel=None):
    """Causal absorbed MLA (optionally restricted to a per-query key set `sel`)."""
    L, H, N = len(q), len(q[0]), len(kv)
    out = [[None] * H for _ in range(L)]
    for h in range(H):
        scores, allowed = [], []
        for i in range(L):
            scores.append([scale * math.fsum(q[i][h][c] * kv[j][c] for c in range(len(kv[j]))) for j in range(N)])
            allowed.append([(j <= N - L + i) and (sel is None or j in sel[i]) for j in range(N)])
        res = attention_rows(scores, [r[:dv] for r in kv], allowed)
        for i in range(L):
            out[i][h] = res[i]
    return out


def indexer_score_exact(qi, kn, wi):
    """Exact rational score sum_h w_h * max(q_h . k, 0) (Fractions)."""
    total = Fraction(0)
    for h in range(len(qi)):
        d = sum((Fraction(a) * Fraction(b) for a, b in zip(qi[h], kn)), Fraction(0))
        if d > 0:
            total += Fraction(wi[h]) * d
    return total


def topk_by_subsets(scores, k):
    """The unique k-subset whose every member beats every non-member.

    "Beats" is the strict total order: higher score, or equal score and lower
    index. Enumerates all subsets, so only for tiny rows. Invisible keys carry
    score None and are never chosen; if fewer than k are visible, all are returned.
    """
    vis = [j for j, s in enumerate(scores) if s is not None]
    kk = min(k, len(vis))

    def beats(a, b):
        return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)

    found = []
    for sub in itertools.combinations(vis, kk):
        rest = [j for j in vis if j not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            found.append(set(sub))
    assert len(found) == 1, "strict total order must give exactly one closed subset"
    return found[0]


def gathered(q_row, kv, idx_row, scale, dv):
    """Attention of one query over an explicitly gathered list of rows.

    The rows named by idx_row are copied out one entry at a time (a repeated
    index appears as often as it is listed; entries outside [0, len(kv)) are
    dropped), every head scores each copy and softmax runs over the copies.
    q_row [H][D] and kv [N][D] are nested lists; returns [H][dv].
    """
    rows = [kv[j] for j in idx_row if 0 <= j < len(kv)]
    if not rows:
        return [[0.0] * dv for _ in q_row]
    out = []
    for qh in q_row:
        scores = [[scale * math.fsum(a * b for a, b in zip(qh, r)) for r in rows]]
        out.append(attention_rows(scores, [r[:dv] for r in rows], [[True] * len(rows)])[0])
    return out
