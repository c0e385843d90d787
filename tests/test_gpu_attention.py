"""GPU parity: dense MLA prefill (non-absorbed fp32/bf16, absorbed bf16) vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from synth import gen_absorbed, gen_nonabsorbed, to_f64
from gpu_util import assert_close, dev, host_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4      # fp32 outputs: max-abs
TOL_BF16 = 2e-2     # bf16 outputs: max-abs


def _nonabs(seed, L, N, H, dtype, scale=1.0):
    g = gen_nonabsorbed(seed, L, N, H=H, dtype=dtype, scale=scale)
    t = {k: dev(v) for k, v in g.items()}
    f = {k: to_f64(v) for k, v in g.items()}
    return t, f


def _run_nonabs(t, causal=True, scale=None):
    out = dm.mla_prefill_dense(t["qn"][None], t["kn"][None], q_rope=t["qr"][None], k_rope=t["kr"][None],
                               v=t["v"][None], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host_f64(out[0])


@pytest.mark.parametrize("L,N,H", [(256, 256, 16), (100, 100, 16), (37, 200, 4), (1, 1, 16), (65, 129, 3)])
def test_nonabsorbed_fp32(L, N, H):
    t, f = _nonabs(1000 if (L, N, H) == (256, 256, 16) else 11 + L, L, N, H, "f32")
    scale = 1 / math.sqrt(192)
    got = _run_nonabs(t)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale)
    assert_close(got, ref, TOL_F32, f"nonabs f32 L={L} N={N} H={H}")


def test_nonabsorbed_fp32_sharpened():
    """Scale x 8 makes softmax peaky, so an off-by-one causal mask or a lost rope term shows up."""
    t, f = _nonabs(21, 96, 96, 16, "f32")
    scale = 8 / math.sqrt(192)
    got = _run_nonabs(t, scale=scale)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale)
    assert_close(got, ref, TOL_F32, "nonabs f32 sharpened")


def test_nonabsorbed_fp32_noncausal():
    t, f = _nonabs(22, 50, 70, 16, "f32")
    scale = 1 / math.sqrt(192)
    got = _run_nonabs(t, causal=False)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale, causal=False)
    assert_close(got, ref, TOL_F32, "nonabs f32 non-causal")


def test_nonabsorbed_fp32_batch_noncausal_more_queries():
    """B = 2, non-causal, more queries than keys (L = 40, N = 23): each entry against the oracle."""
    gs = [gen_nonabsorbed(s, 40, 23, H=5, dtype="f32") for s in (31, 32)]
    t = {k: torch.stack([dev(g[k]) for g in gs]) for k in gs[0]}
    out = dm.mla_prefill_dense(t["qn"], t["kn"], q_rope=t["qr"], k_rope=t["kr"], v=t["v"], causal=False)
    torch.cuda.synchronize()
    for bi, g in enumerate(gs):
        f = {k: to_f64(v) for k, v in g.items()}
        ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192), causal=False)
        assert_close(host_f64(out[bi]), ref, TOL_F32, f"nonabs f32 batch entry {bi}")


def test_nonabsorbed_fp32_long_keys():
    """16 queries at the end of 1000 keys: 63 key blocks, sixteen rounds of the four-way split."""
    t, f = _nonabs(33, 16, 1000, 2, "f32")
    got = _run_nonabs(t)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192))
    assert_close(got, ref, TOL_F32, "nonabs f32 long keys")


def test_nonabsorbed_rope_only_shared_key():
    """Q_nope = 0: only the shared rope key drives the scores."""
    t, f = _nonabs(23, 64, 64, 16, "f32")
    t["qn"].zero_()
    f["qn"][:] = 0
    scale = 1 / math.sqrt(192)
    got = _run_nonabs(t)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale)
    assert_close(got, ref, TOL_F32, "rope-only")


@pytest.mark.parametrize("L,N", [(333, 333), (130, 517)])
def test_nonabsorbed_bf16_small(L, N):
    t, f = _nonabs(30 + L, L, N, 16, "bf16", scale=0.5)
    got = _run_nonabs(t)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192))
    assert_close(got, ref, TOL_BF16, f"nonabs bf16 L={L} N={N}")


@pytest.mark.parametrize("L,N,H", [(1, 1, 16), (37, 200, 4), (129, 129, 3), (256, 1000, 16)])
def test_nonabsorbed_bf16_shapes(L, N, H):
    """Ragged query tiles (not multiples of 128 or 32), odd head counts, L < N, a single key."""
    t, f = _nonabs(40 + L + H, L, N, H, "bf16", scale=0.5)
    got = _run_nonabs(t)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192))
    assert_close(got, ref, TOL_BF16, f"nonabs bf16 L={L} N={N} H={H}")


def test_nonabsorbed_bf16_sharpened_and_first_row():
    """Scale x8 (peaked softmax: a causal off-by-one moves the output far past the tolerance);
    the first query sees only key 0, so its output is V[0] exactly."""
    L = N = 300
    t, f = _nonabs(48, L, N, 16, "bf16", scale=0.5)
    scale = 8 / math.sqrt(192)
    got = _run_nonabs(t, scale=scale)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale)
    assert_close(got, ref, TOL_BF16, "nonabs bf16 sharpened")
    assert np.array_equal(got[0], f["v"][0])


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16), ("f32", TOL_F32)])
@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_nonabsorbed_nonpositive_scale(dtype, tol, scale):
    """A negative scale turns the largest raw score into the smallest weight and zero gives
    equal weights over the visible keys: masking and the running maximum have to follow the
    scaled scores (a causal mask applied before a negative scale would give +inf)."""
    L, N = 160, 200
    t, f = _nonabs(49, L, N, 16, dtype, scale=0.5)
    got = _run_nonabs(t, scale=scale)
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], scale)
    assert_close(got, ref, tol, f"nonabs {dtype} scale={scale}")


def test_nonabsorbed_bf16_noncausal_batch():
    """Non-causal, B = 2: each entry matches the oracle and its own single-sequence call."""
    L, N, H = 70, 333, 16
    gs = [gen_nonabsorbed(60 + e, L, N, H=H, dtype="bf16", scale=0.5) for e in range(2)]
    t = {k: torch.stack([dev(g[k]) for g in gs]) for k in gs[0]}
    out = dm.mla_prefill_dense(t["qn"], t["kn"], q_rope=t["qr"], k_rope=t["kr"], v=t["v"], causal=False)
    one = dm.mla_prefill_dense(t["qn"][1:].contiguous(), t["kn"][1:].contiguous(), q_rope=t["qr"][1:].contiguous(),
                               k_rope=t["kr"][1:].contiguous(), v=t["v"][1:].contiguous(), causal=False)
    torch.cuda.synchronize()
    assert torch.equal(out[1], one[0])
    for e, g in enumerate(gs):
        f = {k: to_f64(v) for k, v in g.items()}
        ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192), causal=False)
        assert_close(host_f64(out[e]), ref, TOL_BF16, f"nonabs bf16 non-causal batch {e}")


def _abs(seed, L, N, H):
    g = gen_absorbed(seed, L, N, H=H)
    return dev(g["q"]), dev(g["kv"]), to_f64(g["q"]), to_f64(g["kv"])


@pytest.mark.parametrize("L,N,H", [(40, 300, 64), (1, 33, 64), (17, 17, 16), (9, 100, 80)])
def test_absorbed_small(L, N, H):
    q, kv, qf, kvf = _abs(40 + L, L, N, H)
    out = dm.mla_prefill_dense(q[None], kv[None])
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(qf, kvf, 1 / math.sqrt(576))
    assert_close(host_f64(out[0]), ref, TOL_BF16, f"absorbed L={L} N={N} H={H}")


@pytest.mark.parametrize("L,N,H", [(50, 300, 64), (300, 100, 16), (7, 1, 80), (130, 33, 64)])
def test_absorbed_noncausal(L, N, H):
    """Non-causal absorbed attention: every query sees all N keys, also with more
    queries than keys (allowed without the causal mask) and a single key."""
    q, kv, qf, kvf = _abs(44 + L, L, N, H)
    out = dm.mla_prefill_dense(q[None], kv[None], causal=False)
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(qf, kvf, 1 / math.sqrt(576), causal=False)
    assert_close(host_f64(out[0]), ref, TOL_BF16, f"absorbed non-causal L={L} N={N} H={H}")


def test_absorbed_sharpened():
    q, kv, qf, kvf = _abs(41, 24, 90, 64)
    scale = 8 / math.sqrt(576)
    out = dm.mla_prefill_dense(q[None], kv[None], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(qf, kvf, scale)
    assert_close(host_f64(out[0]), ref, TOL_BF16, "absorbed sharpened")


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_absorbed_nonpositive_scale(scale):
    """Non-positive scales: the kernel scales and masks before the maximum."""
    q, kv, qf, kvf = _abs(42, 24, 90, 64)
    out = dm.mla_prefill_dense(q[None], kv[None], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(qf, kvf, scale)
    assert_close(host_f64(out[0]), ref, TOL_BF16, f"absorbed scale={scale}")


@pytest.mark.parametrize("scale", [40 / math.sqrt(576), -40 / math.sqrt(576)])
def test_absorbed_wide_score_range(scale):
    """Scores spread over hundreds of log2 units: the first tile's maximum is far below
    (or above) the row's true maximum, so the kernel's second pass against the true
    maximum has to run for these rows."""
    q, kv, qf, kvf = _abs(43, 20, 700, 64)
    out = dm.mla_prefill_dense(q[None], kv[None], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(qf, kvf, scale)
    assert_close(host_f64(out[0]), ref, TOL_BF16, f"absorbed wide range scale={scale:.3f}")


def test_dense_batch():
    """B = 2 (batches take the dense path): each batch entry equals its own single-sequence call."""
    L, N, H = 20, 60, 16
    g1, g2 = gen_absorbed(50, L, N, H=H), gen_absorbed(51, L, N, H=H)
    q = torch.stack([dev(g1["q"]), dev(g2["q"])])
    kv = torch.stack([dev(g1["kv"]), dev(g2["kv"])])
    out = dm.mla_prefill_dense(q, kv)
    o1 = dm.mla_prefill_dense(q[:1].contiguous(), kv[:1].contiguous())
    o2 = dm.mla_prefill_dense(q[1:].contiguous(), kv[1:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out[0], o1[0]) and torch.equal(out[1], o2[0])
    ref = oracle.mla_absorbed(to_f64(g2["q"]), to_f64(g2["kv"]), 1 / math.sqrt(576))
    assert_close(host_f64(out[1]), ref, TOL_BF16, "batch entry 1")
