"""GPU: the decode entry point that allocates nothing, called through the C ABI, gives
the same output as mla_decode_paged (which takes a workspace) on two calls in a row,
the second smaller; a call too large for the fixed scratch is refused up front."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import dsa_sparse_attention_mla_amd as dm
from dsa_sparse_attention_mla_amd import _lib
from synth import bf16_bits, bf16_to_f32
from gpu_util import assert_close, host_f64

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(576)


def _case(seed, lens, page_size, H=64):
    rng = np.random.default_rng(seed)
    maxp = max(1, max((n + page_size - 1) // page_size for n in lens))
    P = sum((n + page_size - 1) // page_size for n in lens) + 2
    pages = bf16_bits(rng.standard_normal((P, page_size, 576), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((len(lens), H, 576), dtype=np.float32))
    perm = rng.permutation(P)
    table = np.zeros((len(lens), maxp), dtype=np.int32)
    pos = 0
    for b, n in enumerate(lens):
        k = (n + page_size - 1) // page_size
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return pages, q, table, np.array(lens, dtype=np.int32)


def _u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _noalloc_abi(q, pages, table, lens, out):
    """Straight through the C ABI (ctypes), as a caller without torch would."""
    B, H, _ = q.shape
    P, ps, _ = pages.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return _lib.lib().mla_decode_paged_noalloc(B, H, P, ps, table.shape[1], p(q), p(pages), p(table), p(lens),
                                               SCALE, p(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_decode_matches_workspace_call():
    assert _lib.lib().mla_decode_paged_noalloc_capacity() == 40 << 20
    results = []
    for seed, lens, ps in ((300, [131072, 70001, 5, 0, 4103, 65536, 1, 90000], 64), (301, [3000, 17], 16)):
        pages, q, table, ln = _case(seed, lens, ps)
        tq, tp, tt, tl = _u16(q), _u16(pages), torch.from_numpy(table).cuda(), torch.from_numpy(ln).cuda()
        out = torch.full((len(lens), 64, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = _noalloc_abi(tq, tp, tt, tl, out)
        assert st == _lib.OK, _lib.status_string(st)
        ref_ws = dm.mla_decode_paged(tq, tp, tt, tl)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any()
        assert torch.equal(out, ref_ws)                          # same kernels, same split: bit-identical
        ref = oracle.mla_decode_paged(bf16_to_f32(q).astype(np.float64), bf16_to_f32(pages).astype(np.float64),
                                      table, ln, SCALE)
        assert_close(host_f64(out), ref, 2e-2, f"no-alloc decode B={len(lens)}", rel_guard=8e-3)
        results.append(out)
    assert results[1].shape[0] == 2                              # the second call was the smaller one


def test_noalloc_decode_refuses_too_large():
    B, H, ps, maxp = 64, 64, 64, 4096                             # 64 sequences x 262144 keys: 2048 records/head
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16, device="cuda")
    pages = torch.zeros((4, ps, 576), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((B, maxp), dtype=torch.int32, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    assert _noalloc_abi(q, pages, table, lens, out) == _lib.WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
