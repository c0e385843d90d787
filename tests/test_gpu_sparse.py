"""GPU parity: sparse absorbed prefill over gathered rows vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from synth import gen_absorbed, gen_topk_indices, to_f64
from gpu_util import assert_close, dev, host_f64

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-2
SCALE = 1 / math.sqrt(576)


def _case(seed, L, N, topk, H=64, pad=0.0):
    g = gen_absorbed(seed, L, N, H=H)
    idx = gen_topk_indices(seed + 7, L, N, topk, pad_frac=pad)
    return dev(g["q"]), dev(g["kv"]), dev(idx), to_f64(g["q"]), to_f64(g["kv"]), idx


@pytest.mark.parametrize("L,N,topk,pad", [(20, 500, 64, 0.0), (33, 1000, 100, 0.2), (5, 40, 48, 0.0), (8, 300, 1, 0.0)])
def test_sparse_small(L, N, topk, pad):
    q, kv, idx, qf, kvf, idxn = _case(60 + L, L, N, topk, pad=pad)
    out = dm.mla_prefill_sparse(q, kv, idx)
    torch.cuda.synchronize()
    ref = oracle.mla_sparse_gather(qf, kvf, idxn, SCALE)
    assert_close(host_f64(out), ref, TOL_BF16, f"sparse L={L} N={N} topk={topk} pad={pad}")
    # the same result as dense attention under the top-k mask
    ref2 = oracle.mla_masked_dense(qf, kvf, idxn, SCALE)
    assert_close(host_f64(out), ref2, TOL_BF16, "sparse vs masked dense")


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_sparse_nonpositive_scale(scale):
    """Non-positive scales with padded index rows: scaled before masking and the maximum."""
    q, kv, idx, qf, kvf, idxn = _case(66, 12, 400, 80, pad=0.2)
    out = dm.mla_prefill_sparse(q, kv, idx, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.mla_sparse_gather(qf, kvf, idxn, scale)
    assert_close(host_f64(out), ref, TOL_BF16, f"sparse scale={scale}")


def test_sparse_full_size_sampled():
    """N = 131072 joined rows, L = 1024 queries, top-k 2048, 64 heads: sampled rows."""
    L, N, topk = 1024, 131072, 2048
    q, kv, idx, qf, kvf, idxn = _case(1004, L, N, topk)
    out = dm.mla_prefill_sparse(q, kv, idx)
    torch.cuda.synchronize()
    got = host_f64(out)
    rows = np.array([0, 1, 511, 512, 1022, 1023])
    ref = oracle.mla_sparse_gather(qf, kvf, idxn, SCALE, rows=rows)
    assert_close(got[rows], ref, TOL_BF16, "sparse 131072 sampled")
    ref2 = oracle.mla_masked_dense(qf, kvf, idxn, SCALE, rows=rows[:2])
    assert_close(got[rows[:2]], ref2, TOL_BF16, "sparse 131072 vs masked dense")
    assert np.isfinite(got).all()


def test_sparse_query_blocks_bit_identical():
    q, kv, idx, *_ = _case(70, 100, 2000, 128)
    outs = [dm.mla_prefill_sparse(q, kv, idx, query_block=b) for b in (1024, 300, 7, 1)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_sparse_permutation_invariance():
    q, kv, idx, qf, kvf, idxn = _case(71, 30, 3000, 256)
    perm = torch.stack([r[torch.randperm(r.numel(), generator=torch.Generator().manual_seed(3)).to(r.device)]
                        for r in idx])
    a = host_f64(dm.mla_prefill_sparse(q, kv, idx))
    b = host_f64(dm.mla_prefill_sparse(q, kv, perm.contiguous()))
    # a different key order changes the fp32 summation order and the running max that the bf16
    # rounding of the softmax weights is taken against: differences are rounding-sized, absolute
    d = np.abs(a - b)
    assert d.max() <= 8e-3 and d.mean() <= 5e-4
    assert_close(b, oracle.mla_sparse_gather(qf, kvf, idxn, SCALE), TOL_BF16, "permuted rows vs oracle")


def test_sparse_short_context_equals_dense():
    """topk covers every visible key: sparse == dense absorbed attention."""
    L, N = 16, 64
    q, kv, _, qf, kvf, _ = _case(72, L, N, N)
    idxn = gen_topk_indices(5, L, N, N)
    out = dm.mla_prefill_sparse(q, kv, dev(idxn))
    dense = dm.mla_prefill_dense(q[None], kv[None])[0]
    torch.cuda.synchronize()
    assert_close(host_f64(out), host_f64(dense), 1e-2, "sparse vs GPU dense")
    assert_close(host_f64(out), oracle.mla_absorbed(qf, kvf, SCALE), TOL_BF16, "short context vs oracle")


def test_sparse_invalid_entries_skipped_and_empty_rows_zero():
    L, N, topk = 6, 50, 8
    q, kv, _, qf, kvf, _ = _case(73, L, N, topk)
    idxn = np.full((L, topk), -1, dtype=np.int32)
    idxn[1, :3] = [0, 7, 49]
    idxn[2, :4] = [5, 60, -9, 11]        # 60 and -9 are out of range: skipped
    idxn[3] = np.arange(8) * 6
    out = host_f64(dm.mla_prefill_sparse(q, kv, dev(idxn)))
    ref = oracle.mla_sparse_gather(qf, kvf, idxn, SCALE)
    assert np.all(out[0] == 0) and np.all(out[4] == 0) and np.all(out[5] == 0)
    assert_close(out, ref, TOL_BF16, "invalid entries")


def test_sparse_repeated_indices_count_per_occurrence():
    """A row listed twice gets two weights, as in a gather (the selection never lists a
    key twice; the masked dense path, a bitmap, would count it once)."""
    L, N, topk = 5, 300, 96
    q, kv, _, qf, kvf, _ = _case(74, L, N, topk)
    rng = np.random.default_rng(75)
    idxn = rng.integers(0, 40, size=(L, topk)).astype(np.int32)   # many repeats
    idxn[4, :] = 17                                                   # one row, 96 times
    out = host_f64(dm.mla_prefill_sparse(q, kv, dev(idxn)))
    ref = oracle.mla_sparse_gather(qf, kvf, idxn, SCALE)
    assert_close(out, ref, TOL_BF16, "repeated indices")
    assert np.allclose(out[4], kvf[17, :512][None, :].repeat(64, axis=0), atol=1e-2)


def test_sparse_inputs_unchanged_outputs_overwritten_repeatable():
    """Inputs are read-only (decode after prefill sees the same cache), every output element is
    written, and repeated runs are bit-identical."""
    q, kv, idx, *_ = _case(74, 64, 4000, 512, pad=0.1)
    snap = [t.clone() for t in (q, kv, idx)]
    out1 = torch.full((64, 64, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    dm.mla_prefill_sparse(q, kv, idx, out=out1)
    out2 = dm.mla_prefill_sparse(q, kv, idx)
    torch.cuda.synchronize()
    for a, b in zip(snap, (q, kv, idx)):
        assert torch.equal(a, b)
    assert not torch.isnan(out1).any()
    assert torch.equal(out1, out2)


# ---- dense attention under the top-k mask (the path the sparse call replaces; the gated case)

def _masked_case(seed, L, N, topk, H=64):
    g = gen_absorbed(seed, L, N, H=H)
    idx = gen_topk_indices(seed + 7, L, N, topk)
    return g, idx


@pytest.mark.parametrize("L,N,topk", [(20, 500, 64), (33, 1000, 100), (5, 40, 48), (1, 37, 4)])
def test_masked_dense_matches_oracle_and_gather(L, N, topk):
    g, idxn = _masked_case(110 + L, L, N, topk)
    q, kv, qf, kvf = dev(g["q"]), dev(g["kv"]), to_f64(g["q"]), to_f64(g["kv"])
    out = host_f64(dm.mla_prefill_masked(q, kv, dev(idxn)))
    ref = oracle.mla_masked_dense(qf, kvf, idxn, SCALE)
    assert_close(out, ref, TOL_BF16, f"masked dense L={L} N={N} topk={topk}")
    gathered = host_f64(dm.mla_prefill_sparse(q, kv, dev(idxn)))
    assert_close(out, gathered, TOL_BF16, "masked dense vs gather")


@pytest.mark.parametrize("L,N,topk,H", [(37, 900, 64, 16), (23, 700, 50, 80), (9, 300, 40, 128)])
def test_masked_dense_other_head_counts(L, N, topk, H):
    """Head counts other than 64: a workgroup's 128 (query, head) rows then span up to
    eight queries (H = 16), or a query's heads span two workgroups (H = 80, 128), so the
    per-wave selection words and causal limits come from different queries."""
    g, idxn = _masked_case(170 + H, L, N, topk, H=H)
    q, kv, qf, kvf = dev(g["q"]), dev(g["kv"]), to_f64(g["q"]), to_f64(g["kv"])
    out = host_f64(dm.mla_prefill_masked(q, kv, dev(idxn)))
    ref = oracle.mla_masked_dense(qf, kvf, idxn, SCALE)
    assert_close(out, ref, TOL_BF16, f"masked dense L={L} N={N} topk={topk} H={H}")
    sparse = host_f64(dm.mla_prefill_sparse(q, kv, dev(idxn)))
    assert_close(sparse, ref, TOL_BF16, f"sparse L={L} N={N} topk={topk} H={H}")


def test_masked_dense_selection_rules():
    """-1 and out-of-range entries ignored, a repeated index selects its key once, a
    selected key past the causal limit stays masked, an empty selection gives zeros."""
    L, N, topk = 6, 70, 8
    g, _ = _masked_case(120, L, N, topk)
    q, kv, qf, kvf = dev(g["q"]), dev(g["kv"]), to_f64(g["q"]), to_f64(g["kv"])
    idxn = np.full((L, topk), -1, dtype=np.int32)
    idxn[0, :3] = [0, 64, 69]            # 69 is past query 0's causal limit (64)
    idxn[1, :4] = [5, 5, 5, 30]           # repeats select once
    idxn[2, :4] = [5, 70, -9, 11]         # out of range: ignored
    idxn[3] = np.arange(8) * 9
    out = host_f64(dm.mla_prefill_masked(q, kv, dev(idxn)))
    ref = oracle.mla_masked_dense(qf, kvf, idxn, SCALE)
    assert np.all(out[4] == 0) and np.all(out[5] == 0)
    assert_close(out, ref, TOL_BF16, "masked selection rules")


def test_masked_dense_wide_score_range():
    """A sharp scale with selections that skip the first key tile for some queries: the
    reference taken from the first tile is empty or far off, so the second pass runs."""
    L, N, topk = 16, 900, 40
    g, idxn = _masked_case(125, L, N, topk)
    idxn[::2] = np.where(idxn[::2] < 64, 64 + (idxn[::2] % 200), idxn[::2])   # nothing in tile 0 or 1
    q, kv, qf, kvf = dev(g["q"]), dev(g["kv"]), to_f64(g["q"]), to_f64(g["kv"])
    scale = 30 / math.sqrt(576)
    out = host_f64(dm.mla_prefill_masked(q, kv, dev(idxn), scale=scale))
    ref = oracle.mla_masked_dense(qf, kvf, idxn, scale)
    assert_close(out, ref, TOL_BF16, "masked dense wide range")


def test_masked_dense_batch():
    L, N, topk, H = 12, 200, 32, 64
    cases = [_masked_case(130 + b, L, N, topk, H) for b in range(2)]
    q = torch.stack([dev(c[0]["q"]) for c in cases])
    kv = torch.stack([dev(c[0]["kv"]) for c in cases])
    idx = torch.stack([dev(c[1]) for c in cases])
    out = dm.mla_prefill_masked(q, kv, idx)
    one = dm.mla_prefill_masked(q[1], kv[1], idx[1])
    torch.cuda.synchronize()
    assert torch.equal(out[1], one)
    for b, (g, idxn) in enumerate(cases):
        ref = oracle.mla_masked_dense(to_f64(g["q"]), to_f64(g["kv"]), idxn, SCALE)
        assert_close(host_f64(out[b]), ref, TOL_BF16, f"masked batch {b}")


def test_dsa_prefill_gated_uses_masked_dense():
    """Below the minimum context the gate sends the chunk to the masked dense path;
    the result matches the oracle's gated prefill."""
    from synth import gen_dsa_prefill
    L, N, topk = 24, 3000, 128
    g = gen_dsa_prefill(140, L, N, H=64)
    t = {k: dev(v) for k, v in g.items()}
    out, idx = dm.dsa_prefill(t["q"], t["kv"], t["q_idx"], t["k_idx"], t["w"], topk)
    torch.cuda.synchronize()
    f = {k: to_f64(v) for k, v in g.items()}
    ref, ref_idx = oracle.dsa_prefill(f["q"], f["kv"], f["q_idx"], f["k_idx"], f["w"], topk, SCALE)
    assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), np.sort(ref_idx, axis=1))
    assert_close(host_f64(out), ref, TOL_BF16, "gated dsa_prefill")


def test_sparse_batched_and_batched_prefill():
    """B = 2 sparse attention equals per-entry calls; dsa_prefill on a batch takes the
    masked path by default (the gate's one-sequence clause) and the sparse path with
    batched_sparse=True, both matching the oracle per entry."""
    from synth import gen_dsa_prefill
    L, N, topk = 16, 3000, 64
    gs = [gen_dsa_prefill(160 + b, L, N, H=64) for b in range(2)]
    t = {k: torch.stack([dev(g[k]) for g in gs]) for k in gs[0]}
    idx = dm.dsa_indexer_topk(t["q_idx"], t["k_idx"], t["w"], topk)
    out = dm.mla_prefill_sparse(t["q"], t["kv"], idx)
    one = dm.mla_prefill_sparse(t["q"][1], t["kv"][1], idx[1])
    torch.cuda.synchronize()
    assert torch.equal(out[1], one)
    out_m, _ = dm.dsa_prefill(t["q"], t["kv"], t["q_idx"], t["k_idx"], t["w"], topk, min_context=1000)
    out_s, idx_s = dm.dsa_prefill(t["q"], t["kv"], t["q_idx"], t["k_idx"], t["w"], topk, min_context=1000,
                                  batched_sparse=True)
    torch.cuda.synchronize()
    for b, g in enumerate(gs):
        f = {k: to_f64(v) for k, v in g.items()}
        ref, ref_idx = oracle.dsa_prefill(f["q"], f["kv"], f["q_idx"], f["k_idx"], f["w"], topk, SCALE,
                                          min_context=1000)
        assert np.array_equal(np.sort(idx_s[b].cpu().numpy(), axis=1), np.sort(ref_idx, axis=1))
        assert_close(host_f64(out_s[b]), ref, TOL_BF16, f"batched sparse prefill entry {b}")
        assert_close(host_f64(out_m[b]), ref, TOL_BF16, f"batched masked prefill entry {b}")
