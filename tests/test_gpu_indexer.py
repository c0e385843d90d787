"""GPU parity: indexer top-k sets must equal the oracle's exactly."""
import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from synth import gen_indexer, gen_indexer_exact, to_f64
from gpu_util import dev, sorted_rows

pytestmark = pytest.mark.gpu


def _run(g, topk, rows=None, block=4096):
    q, k, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    idx, sc = dm.dsa_indexer_topk(q, k, w, topk, block=block, return_scores=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    qf, kf, wf = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    s = oracle.indexer_scores(qf, kf, wf, rows=rows)
    ref = oracle.topk_full(s, topk)
    return idx, sc.cpu().numpy(), ref, s


def _check_rows(idx, ref, rows, what):
    got = sorted_rows(idx[rows])
    exp = sorted_rows(ref)
    bad = [r for r, (a, b) in zip(rows, zip(got, exp)) if a != b]
    print(f"[{what}] rows checked {len(rows)}, mismatching rows {len(bad)}", flush=True)
    assert not bad, f"{what}: rows {bad[:5]} differ"
    # ascending order within rows, -1 padding at the end
    for r in rows:
        row = idx[r]
        v = row[row >= 0]
        assert np.all(np.diff(v) > 0) and np.all(row[len(v):] == -1)


@pytest.mark.parametrize("L,N,topk", [(8, 300, 16), (37, 1000, 64), (5, 5000, 2048), (64, 64, 16), (3, 70000, 100),
                                    (1, 1, 1), (1, 7, 2048), (3, 3, 2)])
def test_indexer_small(L, N, topk):
    g = gen_indexer(80 + L, L, N)
    idx, _, ref, _ = _run(g, topk)
    _check_rows(idx, ref, np.arange(L), f"indexer L={L} N={N} k={topk}")


@pytest.mark.parametrize("L,N,topk", [(16, 2000, 64), (12, 20000, 2048)])
def test_indexer_exact_inputs_ties(L, N, topk):
    """q, k in {-1,0,1}, w multiples of 2^-6: fp32 scores are exact and ties are frequent,
    so the lower-index tie rule decides many keys."""
    g = gen_indexer_exact(90 + L, L, N)
    idx, sc, ref, s = _run(g, topk)
    _check_rows(idx, ref, np.arange(L), f"exact-input indexer L={L} N={N}")


@pytest.mark.parametrize("N,topk", [(5000, 100), (20000, 300)])
def test_indexer_band_over_64_keys(N, topk):
    """150 copies of query 0's k-th key share its score exactly, so the band around the
    k-th score holds more than 64 keys (the refine step's second ranking path) and the
    lower-index rule picks among the copies; N = 20000 runs the sampled-start kernel."""
    L = 2
    g = gen_indexer(130 + topk, L, N)
    s0 = oracle.indexer_scores(to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"]), rows=[0])[0]
    order = np.argsort(-s0[:N - L + 1], kind="stable")        # query 0's visible keys, best first
    star = int(order[topk - 1])
    pool = order[3 * topk:]
    dup = np.random.default_rng(7).choice(pool, 150, replace=False)
    g["k_idx"].data[dup] = g["k_idx"].data[star]
    idx, _, ref, s = _run(g, topk)
    assert int(np.sum(s[0] == s[0][star])) >= 151
    _check_rows(idx, ref, np.arange(L), f"band over 64 keys N={N} k={topk}")


def test_indexer_zero_query_all_ties():
    """q = 0: every visible score is 0, the set is the lowest topk visible indices (exact fallback path)."""
    g = gen_indexer(95, 6, 9000)
    g["q_idx"].data[:] = 0
    idx, _, ref, _ = _run(g, 2048)
    _check_rows(idx, ref, np.arange(6), "zero query")


def test_indexer_sampled_start_moderate_context():
    """Contexts of at least 16384 visible keys start the filter threshold from a scored
    sample of 2048 keys: every row must still equal the oracle."""
    g = gen_indexer(98, 8, 40000)
    idx, sc, ref, s = _run(g, 512)
    _check_rows(idx, ref, np.arange(8), "sampled start L=8 N=40000 k=512")
    # the filter path returns fp32 MFMA estimates, a good share of which differ from
    # the fp32-rounded canonical scores (the exact fallback returns those exactly)
    canon = np.take_along_axis(s, idx.astype(np.int64), axis=1).astype(np.float32)
    assert np.mean(sc != canon) > 0.05


def test_indexer_sampled_start_adversarial():
    """Keys at the sampled positions are scaled by 4, so the sampled start lands far
    above the true k-th score and the lists miss most of the top-k: the refine step
    must detect it and the exact fallback must still return the oracle's sets."""
    L, N, topk, sample = 4, 20000, 2048, 2048      # the 2048 positions include the 1024-key sample's
    g = gen_indexer(99, L, N)
    nv_min = N - L + 1                       # keys visible to every query of the group
    pos = (np.arange(sample, dtype=np.int64) * nv_min) // sample
    kb = g["k_idx"].data
    rows = kb[pos]
    nz = (rows & 0x7F80) != 0
    rows[nz] += 0x0100                        # bf16 exponent + 2: exact multiplication by 4
    kb[pos] = rows
    idx, sc, ref, s = _run(g, topk)
    _check_rows(idx, ref, np.arange(L), "sampled start adversarial")
    # every row went through the exact fallback: its scores are the canonical ones in fp32
    canon = np.take_along_axis(s, idx.astype(np.int64), axis=1).astype(np.float32)
    assert np.array_equal(sc, canon)


@pytest.mark.parametrize("L,N,topk,shift", [(24, 3000, 64, 0.5), (10, 20000, 2048, 0.5),
                                            (8, 40000, 512, 0.5), (8, 40000, 512, 0.9)])
def test_indexer_signed_weights(L, N, topk, shift):
    """Head weights of either sign (w - shift, w ~ U[0,1)): scores can be negative and,
    with shift = 0.9, sum_h w_h ||q_h|| < 0, so an error bound that used w_h rather
    than |w_h| would come out negative. Every row must equal the oracle, on the
    short-context path and on the sampled-start list path (N = 40000)."""
    g = gen_indexer(120 + L, L, N)
    g["w"].data[:] = g["w"].data - np.float32(shift)
    idx, _, ref, s = _run(g, topk)
    assert (s[np.isfinite(s)] < 0).any()
    _check_rows(idx, ref, np.arange(L), f"signed weights L={L} N={N} shift={shift}")


def test_indexer_signed_weights_exact_ties():
    """Exact-input variant with w in [-1, 1) (multiples of 2^-6): negative scores and
    frequent ties, decided by the lower index."""
    g = gen_indexer_exact(130, 12, 20000)
    g["w"].data[:] = np.float32(2.0) * g["w"].data - np.float32(1.0)
    idx, _, ref, _ = _run(g, 2048)
    _check_rows(idx, ref, np.arange(12), "signed exact-input indexer")


def _scale_pow2(t, e):
    """Multiply every nonzero bf16 value of t by 2^e exactly (a shift of the exponent field)."""
    b = t.data
    ex = (b.astype(np.int32) >> 7) & 0xFF
    nz = ex != 0
    assert np.all(ex[nz] + e >= 1) and np.all(ex[nz] + e <= 254), "scaled values leave the bf16 normal range"
    b[nz] = (b[nz].astype(np.int32) + (e << 7)).astype(np.uint16)


@pytest.mark.parametrize("N,eq,ek,ew,what", [
    (9000, 20, 110, 0, "dot products past the fp32 range"),
    (40000, 20, 110, 0, "dot products past the fp32 range, sampled start"),
    (9000, -66, 60, 0, "query squares below the fp32 range, products normal"),
    (9000, -60, -60, 0, "products near and below the fp32 normal range"),
    (9000, 0, 0, 100, "weights of 2^100 (scores still in fp32 range)"),
    (9000, 0, 0, 120, "weights of 2^120 (scores may overflow fp32)"),
])
def test_indexer_extreme_magnitudes(N, eq, ek, ew, what):
    """q, k (and w) scaled by powers of two far outside the range the fp32 filter is
    comfortable in. The canonical fp64 scores only scale, so the set cannot change,
    while the fp32 scores overflow to inf / NaN, or their norms underflow, or products
    flush to zero: the error bound must still hold (norms taken in fp64, an absolute
    term for flushed results) or send the query to the exact fallback. Every row must
    equal the oracle's set and the unscaled inputs' set."""
    L, topk = 6 if N < 16384 else 4, 512
    g = gen_indexer(140, L, N)
    idx0, _, ref0, _ = _run(g, topk)
    _check_rows(idx0, ref0, np.arange(L), f"unscaled, N={N}")
    _scale_pow2(g["q_idx"], eq)
    _scale_pow2(g["k_idx"], ek)
    if ew:
        g["w"].data[:] = g["w"].data * np.float32(2.0 ** ew)
    idx, _, ref, _ = _run(g, topk)
    _check_rows(idx, ref, np.arange(L), f"indexer, {what}")
    assert sorted_rows(idx) == sorted_rows(idx0)


def _eps_rows(g, rows):
    """The per-query error bound the filter's band is built on, recomputed in fp64:
    2.5e-5 * sum_h |w_h| ||q_h|| * max_n ||k_n||."""
    q, k, w = to_f64(g["q_idx"])[rows], to_f64(g["k_idx"]), to_f64(g["w"])[rows]
    kmax = np.sqrt((k * k).sum(axis=1).max())
    return 2.5e-5 * (np.abs(w) * np.sqrt((q * q).sum(axis=2))).sum(axis=1) * kmax


def _check_score_error(g, idx, sc, s, rows, what):
    """|s_hat - s| of every returned key within an eighth of its row's bound: the bound
    holds with room to spare, so the band re-score is what decides near-ties."""
    got_s = np.take_along_axis(s, np.maximum(idx[rows], 0).astype(np.int64), axis=1)
    err = np.where(idx[rows] >= 0, np.abs(sc[rows] - got_s), 0.0).max(axis=1)
    eps = _eps_rows(g, rows)
    print(f"[{what}] max |s_hat - s| = {err.max():.3e}, max ratio to eps = {(err / eps).max():.4f}", flush=True)
    assert np.all(err <= eps / 8)


def test_indexer_full_size_small_config():
    """L = 512, N = 65536, top-k 2048 (blocks of 4096): every row against the oracle."""
    g = gen_indexer(1003, 512, 65536)
    idx, sc, ref, s = _run(g, 2048)
    _check_rows(idx, ref, np.arange(512), "indexer 512 x 65536")
    _check_score_error(g, idx, sc, s, np.arange(512), "score error 512 x 65536")


def test_indexer_block_argument_has_no_effect():
    g = gen_indexer(96, 20, 9000)
    q, k, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    outs = [dm.dsa_indexer_topk(q, k, w, 256, block=b) for b in (4096, 1000, 1)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_indexer_repeatable_and_inputs_unchanged():
    g = gen_indexer(97, 40, 30000)
    q, k, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    snap = [t.clone() for t in (q, k, w)]
    a = dm.dsa_indexer_topk(q, k, w, 2048)
    out = torch.full((40, 2048), -7, dtype=torch.int32, device=q.device)
    dm.dsa_indexer_topk(q, k, w, 2048, out=out)
    torch.cuda.synchronize()
    assert torch.equal(a, out)
    for x, y in zip(snap, (q, k, w)):
        assert torch.equal(x, y)


def test_indexer_batched_equals_per_entry():
    """B = 2: each batch entry's sets equal its own single-sequence call and the oracle."""
    gs = [gen_indexer(150 + b, 12, 3000) for b in range(2)]
    q = torch.stack([dev(g["q_idx"]) for g in gs])
    k = torch.stack([dev(g["k_idx"]) for g in gs])
    w = torch.stack([dev(g["w"]) for g in gs])
    idx = dm.dsa_indexer_topk(q, k, w, 256)
    one = dm.dsa_indexer_topk(q[1], k[1], w[1], 256)
    torch.cuda.synchronize()
    assert torch.equal(idx[1], one)
    for b, g in enumerate(gs):
        s = oracle.indexer_scores(to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"]))
        _check_rows(idx[b].cpu().numpy(), oracle.topk_full(s, 256), np.arange(12), f"batched indexer entry {b}")


def test_indexer_fallback_every_row_full_size():
    """Worst case of the exact fallback at the full workload size: with q = 0 every visible
    score is 0 for all 1024 queries over 131072 keys, so every row fails the coverage
    check and is solved by the fallback from canonical fp64 scores of all its keys; the
    set is the lowest 2048 indices of every row. The call's time is printed (it is the
    cliff a badly placed sampled start costs)."""
    L, N, topk = 1024, 131072, 2048
    g = gen_indexer(1005, L, N)
    g["q_idx"].data[:] = 0
    q, k, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    ws = torch.empty(dm.indexer_workspace_bytes(L, N, topk), dtype=torch.uint8, device="cuda")
    idx = torch.empty((L, topk), dtype=torch.int32, device="cuda")
    dm.dsa_indexer_topk(q, k, w, topk, out=idx, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    dm.dsa_indexer_topk(q, k, w, topk, out=idx, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    print(f"[indexer fallback, all {L} rows of {N} keys] {a.elapsed_time(b):.2f} ms", flush=True)
    want = torch.arange(topk, dtype=torch.int32, device="cuda").expand(L, topk)
    assert torch.equal(idx, want)


def test_indexer_sampled_start_adversarial_full_size():
    """The ×4 sampled-key construction at the full workload (1024 queries, 131072 keys):
    keys at the sampled positions of the first query group are scaled by 4, so its
    sampled start lands far above its true k-th score; the affected rows must come back
    exact through the fallback. The call's time and the number of rows the fallback
    solved (their returned scores are the canonical ones) are printed."""
    L, N, topk, sample, gq = 1024, 131072, 2048, 2048, 8   # the sample this workload takes
    g = gen_indexer(1070, L, N)
    nv_min = N - L + 1                       # keys every query of the first group sees
    pos = (np.arange(sample, dtype=np.int64) * nv_min) // sample
    kb = g["k_idx"].data
    rows = kb[pos]
    nz = (rows & 0x7F80) != 0
    rows[nz] += 0x0100                        # bf16 exponent + 2: exact multiplication by 4
    kb[pos] = rows
    q, k, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    ws = torch.empty(dm.indexer_workspace_bytes(L, N, topk), dtype=torch.uint8, device="cuda")
    idx = torch.empty((L, topk), dtype=torch.int32, device="cuda")
    dm.dsa_indexer_topk(q, k, w, topk, out=idx, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    idx_d, sc_d = dm.dsa_indexer_topk(q, k, w, topk, return_scores=True, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    check = np.unique(np.concatenate([np.arange(2 * gq), [100, 511, 1023]]))
    qf, kf, wf = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    s = oracle.indexer_scores(qf, kf, wf, rows=check)
    ref = oracle.topk_full(s, topk)
    got = idx_d.cpu().numpy()
    _check_rows(got, ref, check, "sampled start adversarial, full size")
    canon = np.take_along_axis(s, got[check].astype(np.int64), axis=1).astype(np.float32)
    fb_rows = int((sc_d.cpu().numpy()[check] == canon).all(axis=1).sum())
    print(f"[indexer adversarial 1024 x 131072] {a.elapsed_time(b):.2f} ms; of the {len(check)} checked rows, "
          f"{fb_rows} came back through the fallback", flush=True)
    assert fb_rows >= gq                      # the first group's rows all needed the fallback
