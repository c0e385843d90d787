"""GPU parity over seeded random shapes: every call against the fp64 oracle on shapes
drawn from the ranges each call supports (sizes below one tile, ragged tails, head
counts, top-k sizes, block arguments, page sizes), beyond the hand-picked cases of
the other test files. The draws are fixed by the seeds, so a failure reproduces."""
import math

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from synth import bf16_bits, bf16_to_f32, gen_absorbed, gen_indexer, gen_nonabsorbed, gen_topk_indices, to_f64
from gpu_util import assert_close, dev, host_f64, sorted_rows

pytestmark = pytest.mark.gpu
TOL_BF16, TOL_F32 = 2e-2, 1e-4


def _loguniform(rng, lo, hi):
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def _indexer_cases(n=10, seed=500):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 25))
        N = max(L, _loguniform(rng, 1, 25000))
        topk = int(rng.choice([1, 3, 17, 64, 200, 512, 1000, 2048, 2560]))
        block = int(rng.choice([1, 5, 4096]))
        out.append((seed + c, L, N, topk, block))
    return out


@pytest.mark.parametrize("seed,L,N,topk,block", _indexer_cases())
def test_random_indexer(seed, L, N, topk, block):
    g = gen_indexer(seed, L, N)
    idx = dm.dsa_indexer_topk(dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"]), topk, block=block)
    torch.cuda.synchronize()
    s = oracle.indexer_scores(to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"]))
    ref = oracle.topk_full(s, topk)
    got = idx.cpu().numpy()
    assert sorted_rows(got) == sorted_rows(ref), f"indexer L={L} N={N} topk={topk} block={block}"
    for row in got:                       # ascending keys, then -1 padding
        v = row[row >= 0]
        assert np.all(np.diff(v) > 0) and np.all(row[len(v):] == -1)


def _sparse_cases(n=8, seed=600):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 31))
        N = max(L, _loguniform(rng, 1, 4000))
        H = int(rng.choice([16, 64, 80, 128]))
        topk = int(rng.integers(1, 701))
        pad = float(rng.choice([0.0, 0.3]))
        out.append((seed + c, L, N, H, topk, pad))
    return out


@pytest.mark.parametrize("seed,L,N,H,topk,pad", _sparse_cases())
def test_random_sparse_and_masked(seed, L, N, H, topk, pad):
    g = gen_absorbed(seed, L, N, H=H)
    idx = gen_topk_indices(seed + 1, L, N, topk, pad_frac=pad)
    q, kv, ix = dev(g["q"]), dev(g["kv"]), dev(idx)
    qf, kvf = to_f64(g["q"]), to_f64(g["kv"])
    scale = 1 / math.sqrt(576)
    out = dm.mla_prefill_sparse(q, kv, ix, query_block=int(np.random.default_rng(seed).integers(1, 1025)))
    torch.cuda.synchronize()
    ref = oracle.mla_sparse_gather(qf, kvf, idx, scale)
    assert_close(host_f64(out), ref, TOL_BF16, f"sparse L={L} N={N} H={H} topk={topk} pad={pad}")
    out_m = dm.mla_prefill_masked(q, kv, ix)
    torch.cuda.synchronize()
    ref_m = oracle.mla_masked_dense(qf, kvf, idx, scale)
    assert_close(host_f64(out_m), ref_m, TOL_BF16, f"masked L={L} N={N} H={H} topk={topk} pad={pad}")


def _absorbed_cases(n=6, seed=700):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 41))
        causal = bool(rng.integers(0, 2))
        N = int(rng.integers(L if causal else 1, 2001))
        H = int(rng.choice([16, 32, 48, 64, 80]))
        out.append((seed + c, L, N, H, causal))
    return out


@pytest.mark.parametrize("seed,L,N,H,causal", _absorbed_cases())
def test_random_absorbed_dense(seed, L, N, H, causal):
    g = gen_absorbed(seed, L, N, H=H)
    out = dm.mla_prefill_dense(dev(g["q"])[None], dev(g["kv"])[None], causal=causal)
    torch.cuda.synchronize()
    ref = oracle.mla_absorbed(to_f64(g["q"]), to_f64(g["kv"]), 1 / math.sqrt(576), causal=causal)
    assert_close(host_f64(out[0]), ref, TOL_BF16, f"absorbed L={L} N={N} H={H} causal={causal}")


def _nonabsorbed_cases(n=8, seed=800):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        dtype = "bf16" if c % 2 == 0 else "f32"
        L = int(rng.integers(1, 301))
        causal = bool(rng.integers(0, 2))
        N = int(rng.integers(L if causal else 1, 701))
        H = int(rng.choice([1, 2, 5, 16]))
        out.append((seed + c, dtype, L, N, H, causal))
    return out


@pytest.mark.parametrize("seed,dtype,L,N,H,causal", _nonabsorbed_cases())
def test_random_nonabsorbed(seed, dtype, L, N, H, causal):
    g = gen_nonabsorbed(seed, L, N, H=H, dtype=dtype, scale=0.5 if dtype == "bf16" else 1.0)
    t = {k: dev(v)[None] for k, v in g.items()}
    out = dm.mla_prefill_dense(t["qn"], t["kn"], q_rope=t["qr"], k_rope=t["kr"], v=t["v"], causal=causal)
    torch.cuda.synchronize()
    f = {k: to_f64(v) for k, v in g.items()}
    ref = oracle.mla_nonabsorbed(f["qn"], f["qr"], f["kn"], f["kr"], f["v"], 1 / math.sqrt(192), causal=causal)
    assert_close(host_f64(out[0]), ref, TOL_BF16 if dtype == "bf16" else TOL_F32,
                 f"non-absorbed {dtype} L={L} N={N} H={H} causal={causal}")


def _decode_cases(n=4, seed=900):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        B = int(rng.integers(1, 6))
        ps = [1, 5, 32, 100][c % 4]
        lens = [int(x) for x in rng.integers(1, 3000, size=B)]
        H = int(rng.choice([16, 64]))
        out.append((seed + c, lens, ps, H))
    return out


@pytest.mark.parametrize("seed,lens,ps,H", _decode_cases())
def test_random_decode(seed, lens, ps, H):
    rng = np.random.default_rng(seed)
    maxp = max((n + ps - 1) // ps for n in lens)
    need = sum((n + ps - 1) // ps for n in lens)
    P = need + 2
    pages = bf16_bits(rng.standard_normal((P, ps, 576), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((len(lens), H, 576), dtype=np.float32))
    perm = rng.permutation(P)
    table = np.zeros((len(lens), maxp), dtype=np.int32)
    pos = 0
    for b, n in enumerate(lens):
        k = (n + ps - 1) // ps
        table[b, :k] = perm[pos:pos + k]
        pos += k
    lens_a = np.asarray(lens, dtype=np.int32)
    as_dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    out = dm.mla_decode_paged(as_dev(q), as_dev(pages), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens_a).cuda())
    torch.cuda.synchronize()
    ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64),
                                  table, lens_a, 1 / math.sqrt(576))
    assert_close(host_f64(out), ref, TOL_BF16, f"decode lens={lens} page={ps} H={H}")
