"""Seeded input generators (no attention or indexer arithmetic lives here).

Recipe: numpy ``default_rng(seed)``; tensors are drawn in the order they are
listed in each function; normal draws are fp32 ``standard_normal`` (times a
stated scale), uniform draws fp32 ``random`` on [0, 1). A bf16 tensor is the
round-to-nearest-even of the fp32 draw, stored as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "to_f64", "Tensor",
    "gen_nonabsorbed", "gen_absorbed", "gen_indexer", "gen_indexer_exact",
    "gen_topk_indices", "gen_dsa_prefill", "CONFIG_SEED", "to_torch",
]

# seed used for the workload shapes listed in the design doc (seed = 1000 + config number)
CONFIG_SEED = {i: 1000 + i for i in range(5)}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by round-to-nearest-even, returned as uint16 bit patterns."""
    # uint32 arithmetic: a carry past bit 31 wraps, and (a mod 2^32) >> 16 equals
    # (a >> 16) mod 2^16, so the result is the same as with wider integers
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> 16) & np.uint32(1)
    return (r >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """A generated tensor: storage array (uint16 for bf16, float32 for fp32) and its dtype name."""
    data: np.ndarray
    dtype: str  # "bf16" or "f32"

    @property
    def shape(self):
        return self.data.shape


def to_f64(t) -> np.ndarray:
    """Exact fp64 view of a generated tensor's values."""
    if isinstance(t, Tensor):
        if t.dtype == "bf16":
            return bf16_to_f32(t.data).astype(np.float64)
        return t.data.astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def _normal(rng, shape, scale, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        return Tensor(bf16_bits(x), "bf16")
    return Tensor(x, "f32")


def gen_nonabsorbed(seed, L, N, H=16, d_nope=128, d_rope=64, d_v=128, dtype="f32", scale=1.0):
    """Non-absorbed MLA inputs, drawn in the order Qn, Qr, Kn, Kr, V.

    Shapes: Qn [L,H,d_nope], Qr [L,H,d_rope], Kn [N,H,d_nope], Kr [N,d_rope]
    (one rope key per position, shared by every head), V [N,H,d_v].
    """
    rng = np.random.default_rng(seed)
    return dict(
        qn=_normal(rng, (L, H, d_nope), scale, dtype),
        qr=_normal(rng, (L, H, d_rope), scale, dtype),
        kn=_normal(rng, (N, H, d_nope), scale, dtype),
        kr=_normal(rng, (N, d_rope), scale, dtype),
        v=_normal(rng, (N, H, d_v), scale, dtype),
    )


def gen_absorbed(seed, L, N, H=64, d=576, scale=1.0):
    """Absorbed MLA inputs in bf16, drawn in the order q, kv.

    q [L,H,d] is the latent-space query (latent part first, rope part last);
    kv [N,d] is the joined latent+rope cache row, one per position.
    """
    rng = np.random.default_rng(seed)
    return dict(q=_normal(rng, (L, H, d), scale, "bf16"), kv=_normal(rng, (N, d), scale, "bf16"))


def gen_indexer(seed, L, N, Hi=32, Di=128):
    """Indexer inputs, drawn in the order q_idx (bf16), k_idx (bf16), w (fp32 U[0,1))."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (L, Hi, Di), 1.0, "bf16")
    k = _normal(rng, (N, Di), 1.0, "bf16")
    w = Tensor(rng.random((L, Hi), dtype=np.float32), "f32")
    return dict(q_idx=q, k_idx=k, w=w)


def gen_indexer_exact(seed, L, N, Hi=32, Di=128, p_zero=0.5):
    """Indexer inputs on which every fp32 evaluation order is exact.

    q and k entries are in {-1, 0, 1} (zero with probability p_zero), w is a
    multiple of 2^-6 in [0, 1). Dot products are small integers and every
    weighted head sum is a multiple of 2^-6 below 2^13, so fp32 arithmetic in
    any order gives the exact value and ties between keys are frequent.
    """
    rng = np.random.default_rng(seed)

    def tern(shape):
        sgn = rng.integers(0, 2, size=shape) * 2 - 1
        nz = rng.random(shape) >= p_zero
        return (sgn * nz).astype(np.float32)

    q = Tensor(bf16_bits(tern((L, Hi, Di))), "bf16")
    k = Tensor(bf16_bits(tern((N, Di))), "bf16")
    w = Tensor((rng.integers(0, 64, size=(L, Hi)) / 64.0).astype(np.float32), "f32")
    return dict(q_idx=q, k_idx=k, w=w)


def gen_dsa_prefill(seed, L, N, H=64, Hi=32, Di=128, d=576):
    """End-to-end DSA prefill inputs from one generator, drawn in the order
    q_idx [L,Hi,Di] (bf16), k_idx [N,Di] (bf16), w [L,Hi] (fp32 U[0,1)),
    q [L,H,d] (bf16), kv [N,d] (bf16). N counts every cached position,
    this chunk's L positions (the last ones) included."""
    rng = np.random.default_rng(seed)
    q_idx = _normal(rng, (L, Hi, Di), 1.0, "bf16")
    k_idx = _normal(rng, (N, Di), 1.0, "bf16")
    w = Tensor(rng.random((L, Hi), dtype=np.float32), "f32")
    q = _normal(rng, (L, H, d), 1.0, "bf16")
    kv = _normal(rng, (N, d), 1.0, "bf16")
    return dict(q_idx=q_idx, k_idx=k_idx, w=w, q=q, kv=kv)


def gen_topk_indices(seed, L, N, topk, causal=True, pad_frac=0.0):
    """Random distinct key indices per query (an index list in the indexer's output format).

    Query i sits at position N - L + i; with causal=True its indices are drawn
    from [0, N - L + i]. A fraction pad_frac of each row is replaced by -1.
    Rows with fewer visible keys than topk hold all visible keys, then -1.
    """
    rng = np.random.default_rng(seed)
    out = np.full((L, topk), -1, dtype=np.int32)
    for i in range(L):
        vis = (N - L + i + 1) if causal else N
        if vis <= topk:
            sel = rng.permutation(vis)
        else:
            sel = rng.choice(vis, size=topk, replace=False)
        out[i, : len(sel)] = sel
        if pad_frac > 0:
            m = rng.random(topk) < pad_frac
            out[i, m] = -1
    return out


def to_torch(t, device="cuda:0"):
    """A generated tensor (or numpy array) as a torch tensor on `device` with the same
    storage bits (bf16 tensors become torch.bfloat16)."""
    import torch
    if isinstance(t, Tensor):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    return torch.from_numpy(np.ascontiguousarray(t)).to(device)
