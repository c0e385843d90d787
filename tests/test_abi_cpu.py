"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import dsa_sparse_attention_mla_amd as dm
from dsa_sparse_attention_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p(4096)       # a fake, 16-byte aligned "device" pointer (never dereferenced)
MIS = ctypes.c_void_p(4098)     # misaligned


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dsa_mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"mla_prefill_dense", "dsa_indexer_topk", "mla_prefill_sparse"} <= names
    lib = dm.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.SIGNATURES) == names
    assert lib.dsa_mla_abi_version() == 1


def _dense(**kw):
    a = dict(mode=0, dtype=1, B=1, L=4, N=8, H=16, q=P, q_rope=P, k=P, k_rope=P, v=P, out=P, scale=0.1, causal=1,
             ws=None, ws_bytes=None, stream=None)
    a.update(kw)
    return dm.lib().mla_prefill_dense(*a.values())


def _indexer(**kw):
    a = dict(B=1, L=4, N=64, Hi=32, Di=128, q=P, k=P, w=P, topk=8, block=4096, idx=P, score=None, ws=None,
             ws_bytes=None, stream=None)
    a.update(kw)
    return dm.lib().dsa_indexer_topk(*a.values())


def _sparse(**kw):
    a = dict(B=1, L=4, N=64, H=64, q=P, kv=P, idx=P, topk=8, scale=0.1, qb=1024, out=P, ws=None, ws_bytes=None,
             stream=None)
    a.update(kw)
    return dm.lib().mla_prefill_sparse(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), _lib.INVALID_ARG), (dict(dtype=5), _lib.INVALID_ARG), (dict(L=-1), _lib.INVALID_ARG),
    (dict(H=0), _lib.INVALID_ARG), (dict(L=9, N=8), _lib.INVALID_ARG), (dict(causal=2), _lib.INVALID_ARG),
    (dict(q=None), _lib.INVALID_ARG), (dict(v=None), _lib.INVALID_ARG), (dict(q=MIS), _lib.INVALID_ARG),
    (dict(scale=float("nan")), _lib.INVALID_ARG), (dict(scale=float("inf")), _lib.INVALID_ARG),
    (dict(mode=1), _lib.INVALID_ARG),                                   # absorbed with rope/v pointers
    (dict(mode=1, q_rope=None, k_rope=None, v=None, dtype=0), _lib.UNSUPPORTED),
    (dict(mode=1, q_rope=None, k_rope=None, v=None, H=24), _lib.UNSUPPORTED),
    (dict(H=65536), _lib.UNSUPPORTED),                                   # non-absorbed: heads past the grid limit
    (dict(mode=1, q_rope=None, k_rope=None, v=None, L=1 << 25, N=1 << 25, H=64), _lib.UNSUPPORTED),  # L*H >= 2^31
    (dict(), _lib.ARCH),                                                 # valid; no gfx950 device here
    (dict(L=0), _lib.OK), (dict(B=0), _lib.OK),                          # empty -> no-op
])
def test_dense_validation(kw, code):
    assert _dense(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(B=2), _lib.WORKSPACE), (dict(Hi=16), _lib.UNSUPPORTED), (dict(Di=64), _lib.UNSUPPORTED),
    (dict(topk=4096), _lib.UNSUPPORTED), (dict(topk=0), _lib.INVALID_ARG), (dict(block=0), _lib.INVALID_ARG),
    (dict(L=65, N=64), _lib.INVALID_ARG), (dict(N=0), _lib.INVALID_ARG), (dict(w=None), _lib.INVALID_ARG),
    (dict(idx=None), _lib.INVALID_ARG), (dict(q=MIS), _lib.INVALID_ARG),
    (dict(), _lib.WORKSPACE),                                            # needs workspace, none given
])
def test_indexer_validation(kw, code):
    assert _indexer(**kw) == code


def test_indexer_workspace_query_and_size_check():
    sz = ctypes.c_size_t(0)
    assert _indexer(L=1024, N=131072, topk=2048, ws_bytes=ctypes.byref(sz)) == _lib.OK
    assert sz.value > 1024 * 2048 * 8
    small = ctypes.c_size_t(sz.value - 1)
    assert _indexer(L=1024, N=131072, topk=2048, ws=P, ws_bytes=ctypes.byref(small)) == _lib.WORKSPACE
    ok = ctypes.c_size_t(sz.value)
    assert _indexer(L=1024, N=131072, topk=2048, ws=P, ws_bytes=ctypes.byref(ok)) == _lib.ARCH
    assert _indexer(L=0, ws=P, ws_bytes=ctypes.byref(ok)) == _lib.OK


@pytest.mark.parametrize("kw,code", [
    (dict(B=2), _lib.ARCH), (dict(H=24), _lib.UNSUPPORTED), (dict(qb=0), _lib.INVALID_ARG),
    (dict(qb=1025), _lib.INVALID_ARG), (dict(topk=0), _lib.INVALID_ARG), (dict(idx=None), _lib.INVALID_ARG),
    (dict(out=MIS), _lib.INVALID_ARG), (dict(scale=float("nan")), _lib.INVALID_ARG),
    (dict(), _lib.ARCH), (dict(L=0), _lib.OK),
])
def test_sparse_validation(kw, code):
    assert _sparse(**kw) == code


def test_dense_and_sparse_need_no_workspace():
    sz = ctypes.c_size_t(123)
    assert _dense(ws_bytes=ctypes.byref(sz)) == _lib.OK and sz.value == 0
    sz = ctypes.c_size_t(123)
    assert _sparse(ws_bytes=ctypes.byref(sz)) == _lib.OK and sz.value == 0


def test_status_strings():
    for s in range(6):
        assert _lib.status_string(s)
    assert _lib.status_string(99) == "unknown status"


def test_gate_helper_matches_predicate():
    assert dm.use_sparse(True, 1, 512, 16384)
    assert not dm.use_sparse(True, 1, 512, 16383)
    assert not dm.use_sparse(True, 2, 512, 131072)
    assert dm.use_sparse(True, 2, 512, 131072, batched=True)        # the one-sequence clause, lifted
    assert not dm.use_sparse(True, 2, 1, 131072, batched=True)
    assert not dm.use_sparse(True, 1, 1, 131072)
    assert not dm.use_sparse(False, 1, 512, 131072)


def _masked(**kw):
    a = dict(B=1, L=4, N=64, H=64, q=P, kv=P, idx=P, topk=8, scale=0.1, out=P, ws=None, ws_bytes=None, stream=None)
    a.update(kw)
    return dm.lib().mla_prefill_masked(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(H=24), _lib.UNSUPPORTED), (dict(topk=0), _lib.INVALID_ARG), (dict(idx=None), _lib.INVALID_ARG),
    (dict(L=65, N=64), _lib.INVALID_ARG), (dict(out=MIS), _lib.INVALID_ARG), (dict(kv=None), _lib.INVALID_ARG),
    (dict(scale=float("nan")), _lib.INVALID_ARG), (dict(), _lib.WORKSPACE), (dict(L=0), _lib.OK),
    (dict(L=1 << 25, N=1 << 25), _lib.UNSUPPORTED),                      # L*H >= 2^31 (64 heads)
])
def test_masked_validation(kw, code):
    assert _masked(**kw) == code


def test_masked_workspace_is_the_bitmaps():
    sz = ctypes.c_size_t(0)
    assert _masked(B=2, L=1024, N=131072, ws_bytes=ctypes.byref(sz)) == _lib.OK
    assert sz.value == 2 * 1024 * (131072 // 32) * 4
    assert dm.masked_workspace_bytes(1, 3, 33) == 3 * 2 * 4
    ok = ctypes.c_size_t(sz.value)
    assert _masked(B=2, L=1024, N=131072, ws=P, ws_bytes=ctypes.byref(ok)) == _lib.ARCH
    small = ctypes.c_size_t(sz.value - 4)
    assert _masked(B=2, L=1024, N=131072, ws=P, ws_bytes=ctypes.byref(small)) == _lib.WORKSPACE


def _decode(**kw):
    a = dict(B=2, H=64, P=16, ps=64, maxp=8, q=P, kv=P, table=P, lens=P, scale=0.1, out=P, ws=None, ws_bytes=None,
             stream=None)
    a.update(kw)
    return dm.lib().mla_decode_paged(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(H=24), _lib.UNSUPPORTED), (dict(ps=0), _lib.INVALID_ARG), (dict(P=0), _lib.INVALID_ARG),
    (dict(maxp=0), _lib.INVALID_ARG), (dict(table=None), _lib.INVALID_ARG), (dict(lens=MIS), _lib.INVALID_ARG),
    (dict(q=MIS), _lib.INVALID_ARG), (dict(scale=float("inf")), _lib.INVALID_ARG), (dict(), _lib.WORKSPACE),
    (dict(ps=1 << 20, maxp=1 << 12), _lib.INVALID_ARG),                 # rows past int32
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_decode_workspace_query():
    sz = ctypes.c_size_t(0)
    assert _decode(ws_bytes=ctypes.byref(sz)) == _lib.OK
    assert sz.value >= 2 * 8 * 64 * 4 + 2 * 64 * 514 * 4
    assert dm.decode_workspace_bytes(2, 64, 16, 64, 8) == sz.value
    ok = ctypes.c_size_t(sz.value)
    assert _decode(ws=P, ws_bytes=ctypes.byref(ok)) == _lib.ARCH
    assert _decode(B=0, ws=P, ws_bytes=ctypes.byref(ok)) == _lib.OK


@pytest.mark.parametrize("kw,code", [
    (dict(grid=0), _lib.INVALID_ARG), (dict(iters=0), _lib.INVALID_ARG), (dict(cyc=None), _lib.INVALID_ARG),
    (dict(sink=None), _lib.INVALID_ARG), (dict(), _lib.ARCH),
])
def test_probe_mfma_validation(kw, code):
    a = dict(grid=256, iters=16, cyc=P, wall=P, sink=P, khz=None, stream=None)
    a.update(kw)
    assert dm.lib().dsa_mla_probe_mfma(*a.values()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), _lib.INVALID_ARG), (dict(nbytes=100), _lib.INVALID_ARG), (dict(src=MIS), _lib.INVALID_ARG),
    (dict(dst=None), _lib.INVALID_ARG), (dict(grid=0), _lib.INVALID_ARG), (dict(nbytes=0), _lib.OK),
    (dict(), _lib.ARCH),
])
def test_probe_stream_validation(kw, code):
    a = dict(mode=0, src=P, dst=P, nbytes=1 << 20, grid=64, stream=None)
    a.update(kw)
    assert dm.lib().dsa_mla_probe_stream(*a.values()) == code
