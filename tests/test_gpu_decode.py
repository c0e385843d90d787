"""GPU parity: one decode step over a paged joined cache vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from synth import bf16_bits, bf16_to_f32, gen_dsa_prefill, to_f64
from gpu_util import assert_close, dev, host_f64, sorted_rows

pytestmark = pytest.mark.gpu
TOL_BF16 = 2e-2
SCALE = 1 / math.sqrt(576)


def _paged_case(seed, lens, page_size, H=64, spare_pages=3):
    """Random bf16 pages; each sequence's pages are scattered over the pool in random order."""
    rng = np.random.default_rng(seed)
    maxp = max(1, max((n + page_size - 1) // page_size for n in lens))
    need = sum((n + page_size - 1) // page_size for n in lens)
    P = need + spare_pages
    pages = bf16_bits(rng.standard_normal((P, page_size, 576), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((len(lens), H, 576), dtype=np.float32))
    perm = rng.permutation(P)
    table = np.zeros((len(lens), maxp), dtype=np.int32)
    pos = 0
    for b, n in enumerate(lens):
        k = (n + page_size - 1) // page_size
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return pages, q, table, np.asarray(lens, dtype=np.int32)


def _run(pages, q, table, lens):
    out = dm.mla_decode_paged(dev_u16(q), dev_u16(pages), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    return host_f64(out)


def dev_u16(a):
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("page_size", [16, 48, 7])
def test_decode_ragged_batch(page_size):
    """Lengths 0, 1, around a page and a tile, and long; pages scattered; page sizes that
    are not multiples of the 32-key tile, so tiles straddle pages."""
    lens = [0, 1, 63, 64, 65, 1000, 4103]
    pages, q, table, ln = _paged_case(200 + page_size, lens, page_size)
    got = _run(pages, q, table, ln)
    ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64), table,
                                  ln, SCALE)
    assert np.all(got[0] == 0)
    assert_close(got, ref, TOL_BF16, f"paged decode page_size={page_size}")


def test_decode_long_contexts():
    lens = [131072, 70001]
    pages, q, table, ln = _paged_case(210, lens, 256, spare_pages=1)
    got = _run(pages, q, table, ln)
    ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64), table,
                                  ln, SCALE)
    assert_close(got, ref, TOL_BF16, "paged decode 131072 / 70001")


def test_decode_one_sequence_many_splits():
    """B = 1 over 130999 keys: the keys split 256 ways, the last split holds only part of
    a tile."""
    lens = [130999]
    pages, q, table, ln = _paged_case(215, lens, 64, spare_pages=2)
    got = _run(pages, q, table, ln)
    ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64), table,
                                  ln, SCALE)
    assert_close(got, ref, TOL_BF16, "paged decode, one sequence of 130999 keys")


def test_decode_more_splits_than_one_combine_pass():
    """B = 1 over 1060001 keys (splits of 4096 keys, the longest): 259 splits, more than
    the combine's 256 per pass. The table maps the 4141 logical pages onto 40 physical
    ones in random order (a page may serve several positions), so the pool stays small."""
    n, ps, P, H = 1_060_001, 256, 40, 16
    rng = np.random.default_rng(216)
    pages = bf16_bits(rng.standard_normal((P, ps, 576), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((1, H, 576), dtype=np.float32))
    table = rng.integers(0, P, size=(1, (n + ps - 1) // ps)).astype(np.int32)
    ln = np.array([n], dtype=np.int32)
    got = _run(pages, q, table, ln)
    ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64), table,
                                  ln, SCALE)
    assert_close(got, ref, TOL_BF16, "paged decode, one sequence of 1060001 keys")


def test_decode_page_outside_pool_counts_as_absent():
    lens = [300]
    pages, q, table, ln = _paged_case(220, lens, 32)
    table[0, 2] = 10_000                          # rows 64..95 point outside the pool
    got = _run(pages, q, table, ln)
    keep = [n for n in range(300) if n // 32 != 2]
    pf = bf16_to_f32(pages).astype(np.float64)
    rows = np.stack([pf[table[0, n // 32], n % 32] for n in keep])
    ref = oracle.mla_absorbed(bf16_to_f32(q[0]).astype(np.float64)[None], rows, SCALE)[0]
    assert_close(got[0], ref, TOL_BF16, "absent page")


def test_decode_after_sparse_prefill():
    """The pages' flow: a chunk is prefilled on the sparse path, then the next token
    decodes over the same cache laid out in pages."""
    L, N, topk, ps = 64, 20000, 512, 64
    g = gen_dsa_prefill(230, L, N, H=64)
    t = {k: dev(v) for k, v in g.items()}
    out, idx = dm.dsa_prefill(t["q"], t["kv"], t["q_idx"], t["k_idx"], t["w"], topk, min_context=16384)
    f = {k: to_f64(v) for k, v in g.items()}
    rows = [0, L // 2, L - 1]
    ref_p, ref_idx = oracle.dsa_prefill(f["q"], f["kv"], f["q_idx"], f["k_idx"], f["w"], topk, SCALE,
                                        min_context=16384, rows=rows)
    assert sorted_rows(idx.cpu().numpy()[rows]) == sorted_rows(ref_idx[rows])   # the selection itself
    assert_close(host_f64(out)[rows], ref_p, TOL_BF16, "sparse prefill rows")
    # next token: its key row is appended at position N; the cache goes into shuffled pages
    rng = np.random.default_rng(231)
    new_row = bf16_bits(rng.standard_normal((1, 576), dtype=np.float32))
    q_dec = bf16_bits(rng.standard_normal((1, 64, 576), dtype=np.float32))
    cache = np.concatenate([g["kv"].data, new_row])                  # [N+1, 576] bf16 bits
    n = N + 1
    npg = (n + ps - 1) // ps
    padded = np.zeros((npg * ps, 576), dtype=np.uint16)
    padded[:n] = cache
    perm = rng.permutation(npg)
    pool = np.zeros((npg, ps, 576), dtype=np.uint16)
    pool[perm] = padded.reshape(npg, ps, 576)
    got = _run(pool, q_dec, perm[None].astype(np.int32), np.array([n], dtype=np.int32))
    ref = oracle.mla_absorbed(bf16_to_f32(q_dec).astype(np.float64), bf16_to_f32(cache).astype(np.float64), SCALE)
    assert_close(got, ref, TOL_BF16, "decode after sparse prefill")
