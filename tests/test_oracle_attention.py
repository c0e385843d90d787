"""Pins for the attention oracle (CPU only).

Each pin checks the oracle against something other than its own formula:
hand-worked values, closed forms, a library attention routine (torch's
scaled_dot_product_attention on CPU in float64), linear-algebra identities and
pure-Python brute force. tests/test_oracle_mutations.py plants plausible
mistakes in copies of the oracle and checks that these pins catch them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nonabs_inputs(rng, L, N, H=3, dn=8, dr=4, dv=5):
    return (rng.standard_normal((L, H, dn)), rng.standard_normal((L, H, dr)),
            rng.standard_normal((N, H, dn)), rng.standard_normal((N, dr)),
            rng.standard_normal((N, H, dv)))


def _sdpa(q, k, v, allowed, scale):
    """torch SDPA in float64 on the CPU: q [H,L,D], k [H,N,D], v [H,N,Dv], allowed [L,N]."""
    with torch.no_grad():
        return torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(allowed), scale=scale).numpy()


# ---- pins as reusable checks (the mutation tests call them on planted mistakes) ----

def pin_nonabs_golden(fn):
    g = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    out = fn(*(np.array(g[k], dtype=np.float64) for k in ("qn", "qr", "kn", "kr", "v")), g["scale"])
    return np.allclose(out, np.array(g["out"]), rtol=0, atol=1e-14)


def pin_nonabs_first_query(fn, rng):
    qn, qr, kn, kr, v = _nonabs_inputs(rng, 6, 6)
    out = fn(qn, qr, kn, kr, v, 0.37)
    return np.array_equal(out[0], v[0])


def pin_nonabs_zero_query_prefix_mean(fn, rng):
    L, N = 5, 9
    qn, qr, kn, kr, v = _nonabs_inputs(rng, L, N)
    out = fn(np.zeros_like(qn), np.zeros_like(qr), kn, kr, v, 1.0)
    csum = np.cumsum(v, axis=0)
    ref = np.stack([csum[N - L + i] / (N - L + i + 1) for i in range(L)])
    return np.allclose(out, ref, rtol=0, atol=1e-13)


def pin_nonabs_vs_sdpa(fn, rng, L=7, N=11):
    """MLA equals standard attention with head dim Dn+Dr over [Qn|Qr] and [Kn|Kr broadcast]."""
    qn, qr, kn, kr, v = _nonabs_inputs(rng, L, N)
    H = qn.shape[1]
    scale = 1 / np.sqrt(qn.shape[2] + qr.shape[2])
    q = np.concatenate([qn, qr], axis=2).transpose(1, 0, 2).copy()
    k = np.concatenate([kn, np.broadcast_to(kr[:, None, :], (N, H, kr.shape[1]))], axis=2).transpose(1, 0, 2).copy()
    allowed = np.arange(N)[None, :] <= (N - L + np.arange(L))[:, None]
    ref = _sdpa(q, k, v.transpose(1, 0, 2).copy(), allowed, scale).transpose(1, 0, 2)
    return np.allclose(fn(qn, qr, kn, kr, v, scale), ref, rtol=0, atol=1e-12)


def pin_nonabs_rope_only(fn, rng):
    """Q_nope = 0: only the shared rope key drives the scores, identically for every head."""
    L, N = 4, 8
    qn, qr, kn, kr, v = _nonabs_inputs(rng, L, N)
    qr[:] = qr[:, :1, :]                      # same rope query in every head
    out = fn(np.zeros_like(qn), qr, kn, kr, v, 0.5)
    H = qn.shape[1]
    allowed = np.arange(N)[None, :] <= (N - L + np.arange(L))[:, None]
    q = np.broadcast_to(qr.transpose(1, 0, 2), (H, L, qr.shape[2])).copy()
    k = np.broadcast_to(kr[None], (H, N, kr.shape[1])).copy()
    ref = _sdpa(q, k, v.transpose(1, 0, 2).copy(), allowed, 0.5).transpose(1, 0, 2)
    return np.allclose(out, ref, rtol=0, atol=1e-12)


def pin_nonabs_brute(fn, rng):
    L, N = 3, 5
    qn, qr, kn, kr, v = _nonabs_inputs(rng, L, N, H=2, dn=3, dr=2, dv=2)
    ref = np.array(brute.nonabsorbed(qn.tolist(), qr.tolist(), kn.tolist(), kr.tolist(), v.tolist(), 0.8))
    return np.allclose(fn(qn, qr, kn, kr, v, 0.8), ref, rtol=0, atol=1e-12)


def pin_absorption_identity(fn_abs, rng):
    """Absorbed attention with q_lat = W_UK^T q_nope and V = W_UV c equals the non-absorbed form."""
    L, N, H, dl, dn, dr, dv = 5, 9, 3, 12, 6, 4, 7
    c = rng.standard_normal((N, dl))
    kr = rng.standard_normal((N, dr))
    w_uk = rng.standard_normal((H, dn, dl))
    w_uv = rng.standard_normal((H, dv, dl))
    qn = rng.standard_normal((L, H, dn))
    qr = rng.standard_normal((L, H, dr))
    kn = np.einsum("hdl,nl->nhd", w_uk, c)
    v = np.einsum("hdl,nl->nhd", w_uv, c)
    ref = oracle.mla_nonabsorbed(qn, qr, kn, kr, v, 0.3)
    q_lat = np.einsum("hdl,ihd->ihl", w_uk, qn)
    q_abs = np.concatenate([q_lat, qr], axis=2)
    rows = np.concatenate([c, kr], axis=1)
    o_lat = fn_abs(q_abs, rows, 0.3, dv=dl)
    out = np.einsum("hdl,ihl->ihd", w_uv, o_lat)
    return np.allclose(out, ref, rtol=0, atol=1e-10)


def pin_absorbed_vs_sdpa(fn_abs, rng, L=6, N=13):
    """Absorbed attention is multi-query attention with K = row, V = row[:dv] broadcast to all heads."""
    H, D, dv = 4, 10, 7
    q = rng.standard_normal((L, H, D))
    kv = rng.standard_normal((N, D))
    allowed = np.arange(N)[None, :] <= (N - L + np.arange(L))[:, None]
    ref = _sdpa(q.transpose(1, 0, 2).copy(), np.broadcast_to(kv, (H, N, D)).copy(),
                np.broadcast_to(kv[:, :dv], (H, N, dv)).copy(), allowed, 0.25).transpose(1, 0, 2)
    return np.allclose(fn_abs(q, kv, 0.25, dv=dv), ref, rtol=0, atol=1e-12)


def pin_absorbed_brute(fn_abs, rng):
    L, N, H, D, dv = 3, 6, 2, 4, 3
    q = rng.standard_normal((L, H, D))
    kv = rng.standard_normal((N, D))
    ref = np.array(brute.absorbed(q.tolist(), kv.tolist(), 0.6, dv))
    return np.allclose(fn_abs(q, kv, 0.6, dv=dv), ref, rtol=0, atol=1e-12)


# ---- tests ----

def test_nonabsorbed_hand_example():
    assert pin_nonabs_golden(oracle.mla_nonabsorbed)


def test_nonabsorbed_first_query_is_first_value(rng):
    assert pin_nonabs_first_query(oracle.mla_nonabsorbed, rng)


def test_nonabsorbed_zero_query_is_prefix_mean(rng):
    assert pin_nonabs_zero_query_prefix_mean(oracle.mla_nonabsorbed, rng)


@pytest.mark.parametrize("L,N", [(7, 11), (9, 9), (1, 5)])
def test_nonabsorbed_matches_library_attention(rng, L, N):
    assert pin_nonabs_vs_sdpa(oracle.mla_nonabsorbed, rng, L, N)


def test_nonabsorbed_rope_key_shared(rng):
    assert pin_nonabs_rope_only(oracle.mla_nonabsorbed, rng)


def test_nonabsorbed_brute_force(rng):
    assert pin_nonabs_brute(oracle.mla_nonabsorbed, rng)


def test_nonabsorbed_rows_subset(rng):
    qn, qr, kn, kr, v = _nonabs_inputs(rng, 8, 12)
    full = oracle.mla_nonabsorbed(qn, qr, kn, kr, v, 0.4)
    part = oracle.mla_nonabsorbed(qn, qr, kn, kr, v, 0.4, rows=[0, 5, 7])
    assert np.array_equal(part, full[[0, 5, 7]])


def test_absorption_identity(rng):
    assert pin_absorption_identity(oracle.mla_absorbed, rng)


@pytest.mark.parametrize("L,N", [(6, 13), (5, 5)])
def test_absorbed_matches_library_attention(rng, L, N):
    assert pin_absorbed_vs_sdpa(oracle.mla_absorbed, rng, L, N)


def test_absorbed_brute_force(rng):
    assert pin_absorbed_brute(oracle.mla_absorbed, rng)


def test_causal_rejects_more_queries_than_keys(rng):
    with pytest.raises(ValueError):
        oracle.visible_mask(5, 4)
