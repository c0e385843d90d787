"""Python wrappers of the three C entry points (argument marshalling only)."""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import check, lib

SPARSE_PREFILL_DEFAULT = True
SPARSE_PREFILL_MIN_CONTEXT_DEFAULT = 16384


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device):
    """The library launches on the current HIP device: make it the tensors' device
    for the call (on a host with several GPUs the current one may be another)."""
    return torch.cuda.device(device)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_out(t, name, dtype, shape, device):
    """A caller-supplied output buffer: exact dtype, shape and device, contiguous. The
    kernels write every element of the expected shape, so a smaller or differently laid
    out buffer would be written past its end; it is refused before anything launches."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _need_workspace(t, nbytes, device):
    """A caller-supplied workspace: a contiguous 1-D uint8 device tensor of at least nbytes."""
    _need(t, "workspace", torch.uint8, 1)
    if t.device != device:
        raise ValueError(f"workspace must be on {device}, got {t.device}")
    if t.numel() < nbytes:
        raise ValueError(f"workspace holds {t.numel()} bytes, {nbytes} needed")


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(query, device):
    size = ctypes.c_size_t(0)
    check(query(None, ctypes.byref(size)), "workspace query")
    if size.value == 0:
        return None, None
    ws = torch.empty(size.value, dtype=torch.uint8, device=device)
    return ws, size


def mla_prefill_dense(q, k, *, q_rope=None, k_rope=None, v=None, scale=None, causal=True, out=None):
    """Dense causal MLA prefill.

    Non-absorbed (q_rope, k_rope, v given): q [B,L,H,128], q_rope [B,L,H,64],
    k [B,N,H,128], k_rope [B,N,64], v [B,N,H,128]; fp32 or bf16; out [B,L,H,128].
    Absorbed (q_rope, k_rope, v omitted): q [B,L,H,576], k = kv [B,N,576] bf16;
    out [B,L,H,512]. scale defaults to 1/sqrt(query width).
    """
    absorbed = q_rope is None and k_rope is None and v is None
    dtype = q.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", dtype, 4)
    _need(k, "k", dtype, 3 if absorbed else 4)
    B, L, H, D = q.shape
    N = k.shape[1]
    if absorbed:
        if D != 576 or k.shape != (B, N, 576):
            raise ValueError("absorbed mode needs q [B,L,H,576] and kv [B,N,576]")
        dv = 512
        if scale is None:
            scale = 1.0 / math.sqrt(576)
    else:
        _need(q_rope, "q_rope", dtype, 4)
        _need(k_rope, "k_rope", dtype, 3)
        _need(v, "v", dtype, 4)
        if (D != 128 or q_rope.shape != (B, L, H, 64) or k.shape != (B, N, H, 128)
                or k_rope.shape != (B, N, 64) or v.shape != (B, N, H, 128)):
            raise ValueError("non-absorbed shapes must be q [B,L,H,128], q_rope [B,L,H,64], k [B,N,H,128], "
                             "k_rope [B,N,64], v [B,N,H,128]")
        dv = 128
        if scale is None:
            scale = 1.0 / math.sqrt(192)
    _same_device(q.device, k=k, q_rope=q_rope, k_rope=k_rope, v=v)
    if out is None:
        out = torch.empty((B, L, H, dv), dtype=dtype, device=q.device)
    else:
        _need_out(out, "out", dtype, (B, L, H, dv), q.device)
    with _on(q.device):
        st = lib().mla_prefill_dense(
            _lib.MODE_ABSORBED if absorbed else _lib.MODE_NONABSORBED,
            _lib.BF16 if dtype == torch.bfloat16 else _lib.F32,
            B, L, N, H, _ptr(q), _ptr(q_rope), _ptr(k), _ptr(k_rope), _ptr(v), _ptr(out),
            float(scale), 1 if causal else 0, None, None, _stream(q.device))
    check(st, "mla_prefill_dense")
    return out


def indexer_workspace_bytes(L, N, topk, block=4096, Hi=32, Di=128):
    """Workspace bytes dsa_indexer_topk needs for these sizes."""
    size = ctypes.c_size_t(0)
    p = ctypes.c_void_p(256)
    check(lib().dsa_indexer_topk(1, L, N, Hi, Di, p, p, p, int(topk), int(block), p, None, None,
                                 ctypes.byref(size), None), "dsa_indexer_topk (workspace query)")
    return size.value


def dsa_indexer_topk(q_idx, k_idx, w, topk, *, block=4096, return_scores=False, out=None, workspace=None):
    """Exact indexer top-k. q_idx [L,32,128] bf16, k_idx [N,128] bf16, w [L,32] fp32
    (or with a leading batch dimension B on all three).

    Returns idx [L,topk] (or [B,L,topk]) int32 (ascending key order, -1 padded), and
    the fp32 scores of the returned keys when return_scores is set. `workspace` (a
    uint8 device tensor of at least indexer_workspace_bytes, which does not depend on
    B) avoids a per-call allocation.
    """
    batched = q_idx.dim() == 4
    if not batched:
        q_idx, k_idx, w = q_idx[None], k_idx[None], w[None]
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 3)
    B, L, Hi, Di = q_idx.shape
    N = k_idx.shape[1]
    if k_idx.shape[0] != B or k_idx.shape[2] != Di or w.shape != (B, L, Hi):
        raise ValueError("shapes must be q_idx [B,L,Hi,Di], k_idx [B,N,Di], w [B,L,Hi]")
    dev = q_idx.device
    _same_device(dev, k_idx=k_idx, w=w)
    if out is not None:
        _need_out(out, "out", torch.int32, (B, L, topk) if batched else (L, topk), dev)
        idx = out if batched else out[None]
    else:
        idx = torch.empty((B, L, topk), dtype=torch.int32, device=dev)
    scores = torch.empty((B, L, topk), dtype=torch.float32, device=dev) if return_scores else None

    def call(ws, ws_bytes):
        with _on(dev):
            return lib().dsa_indexer_topk(B, L, N, Hi, Di, _ptr(q_idx), _ptr(k_idx), _ptr(w), int(topk),
                                          int(block), _ptr(idx), _ptr(scores), ws, ws_bytes, _stream(dev))

    if workspace is not None:
        _need_workspace(workspace, indexer_workspace_bytes(L, N, topk, block, Hi, Di), dev)
        ws, size = workspace, ctypes.c_size_t(workspace.numel())
    else:
        ws, size = _workspace(call, dev)
    check(call(_ptr(ws), None if size is None else ctypes.byref(size)), "dsa_indexer_topk")
    if not batched:
        idx = idx[0]
        scores = scores[0] if scores is not None else None
    return (idx, scores) if return_scores else idx


def mla_prefill_sparse(q, kv, idx, *, scale=None, query_block=1024, out=None):
    """Sparse absorbed prefill. q [L,H,576] bf16, kv [N,576] bf16, idx [L,topk] int32
    -> out [L,H,512] bf16 (or all with a leading batch dimension B)."""
    batched = q.dim() == 4
    if not batched:
        q, kv, idx = q[None], kv[None], idx[None]
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    B, L, H, D = q.shape
    N = kv.shape[1]
    if D != 576 or kv.shape[0] != B or kv.shape[2] != 576 or idx.shape[:2] != (B, L):
        raise ValueError("shapes must be q [B,L,H,576], kv [B,N,576], idx [B,L,topk]")
    if scale is None:
        scale = 1.0 / math.sqrt(576)
    _same_device(q.device, kv=kv, idx=idx)
    if out is None:
        out = torch.empty((B, L, H, 512), dtype=torch.bfloat16, device=q.device)
    else:
        _need_out(out, "out", torch.bfloat16, (B, L, H, 512) if batched else (L, H, 512), q.device)
        out = out if batched else out[None]
    with _on(q.device):
        st = lib().mla_prefill_sparse(B, L, N, H, _ptr(q), _ptr(kv), _ptr(idx), idx.shape[2], float(scale),
                                      int(query_block), _ptr(out), None, None, _stream(q.device))
    check(st, "mla_prefill_sparse")
    return out if batched else out[0]


def masked_workspace_bytes(B: int, L: int, N: int) -> int:
    """Workspace of mla_prefill_masked (the selection bitmaps)."""
    n = ctypes.c_size_t(0)
    p = ctypes.c_void_p(256)                # placeholder pointers: a size query reads nothing
    check(lib().mla_prefill_masked(B, L, N, 16, p, p, p, 1, 1.0, p, None, ctypes.byref(n), None),
          "mla_prefill_masked (workspace query)")
    return n.value


def mla_prefill_masked(q, kv, idx, *, scale=None, out=None, workspace=None):
    """Dense absorbed prefill under each query's top-k selection (the gated path).

    q [L,H,576] or [B,L,H,576] bf16, kv [N,576] or [B,N,576] bf16, idx [L,topk] or
    [B,L,topk] int32 -> out [L,H,512] or [B,L,H,512] bf16.
    """
    batched = q.dim() == 4
    if not batched:
        q, kv, idx = q[None], kv[None], idx[None]
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    B, L, H, D = q.shape
    N = kv.shape[1]
    if D != 576 or kv.shape[0] != B or kv.shape[2] != 576 or idx.shape[:2] != (B, L):
        raise ValueError("shapes must be q [B,L,H,576], kv [B,N,576], idx [B,L,topk]")
    if scale is None:
        scale = 1.0 / math.sqrt(576)
    _same_device(q.device, kv=kv, idx=idx)
    if out is None:
        out = torch.empty((B, L, H, 512), dtype=torch.bfloat16, device=q.device)
    else:
        _need_out(out, "out", torch.bfloat16, (B, L, H, 512) if batched else (L, H, 512), q.device)
        if not batched:
            out = out[None]
    nbytes = masked_workspace_bytes(B, L, N)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _need_workspace(workspace, nbytes, q.device)
    n = ctypes.c_size_t(workspace.numel())
    with _on(q.device):
        st = lib().mla_prefill_masked(B, L, N, H, _ptr(q), _ptr(kv), _ptr(idx), idx.shape[2], float(scale),
                                      _ptr(out), _ptr(workspace), ctypes.byref(n), _stream(q.device))
    check(st, "mla_prefill_masked")
    return out if batched else out[0]


def decode_workspace_bytes(B: int, H: int, num_pages: int, page_size: int, max_pages: int) -> int:
    """Workspace of mla_decode_paged (row lists and split partials)."""
    n = ctypes.c_size_t(0)
    p = ctypes.c_void_p(256)                # placeholder pointers: a size query reads nothing
    check(lib().mla_decode_paged(B, H, num_pages, page_size, max_pages, p, p, p, p, 1.0, p, None, ctypes.byref(n),
                                 None), "mla_decode_paged (workspace query)")
    return n.value


def mla_decode_paged(q, kv_pages, page_table, seq_lens, *, scale=None, out=None, workspace=None):
    """One decode step over a paged joined cache.

    q [B,H,576] bf16, kv_pages [num_pages,page_size,576] bf16, page_table [B,max_pages]
    int32, seq_lens [B] int32 -> out [B,H,512] bf16.
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pages, "kv_pages", torch.bfloat16, 3)
    _need(page_table, "page_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, H, D = q.shape
    P, ps, D2 = kv_pages.shape
    if D != 576 or D2 != 576 or page_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shapes must be q [B,H,576], kv_pages [P,page_size,576], page_table [B,max_pages], "
                         "seq_lens [B]")
    maxp = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(576)
    _same_device(q.device, kv_pages=kv_pages, page_table=page_table, seq_lens=seq_lens)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q.device)
    else:
        _need_out(out, "out", torch.bfloat16, (B, H, 512), q.device)
    nbytes = decode_workspace_bytes(B, H, P, ps, maxp)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _need_workspace(workspace, nbytes, q.device)
    n = ctypes.c_size_t(workspace.numel())
    with _on(q.device):
        st = lib().mla_decode_paged(B, H, P, ps, maxp, _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                                    float(scale), _ptr(out), _ptr(workspace), ctypes.byref(n), _stream(q.device))
    check(st, "mla_decode_paged")
    return out


def mla_decode_paged_noalloc(q, kv_pages, page_table, seq_lens, *, scale=None, out):
    """mla_decode_paged without a workspace: the split partials go to the library's fixed
    device scratch (for callers that cannot allocate). `out` [B,H,512] bf16 is required.
    Calls on one device must not overlap in time (they share the scratch)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pages, "kv_pages", torch.bfloat16, 3)
    _need(page_table, "page_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, H, D = q.shape
    P, ps, D2 = kv_pages.shape
    if D != 576 or D2 != 576 or page_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shapes must be q [B,H,576], kv_pages [P,page_size,576], page_table [B,max_pages], "
                         "seq_lens [B]")
    _same_device(q.device, kv_pages=kv_pages, page_table=page_table, seq_lens=seq_lens)
    _need_out(out, "out", torch.bfloat16, (B, H, 512), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(576)
    with _on(q.device):
        st = lib().mla_decode_paged_noalloc(B, H, P, ps, page_table.shape[1], _ptr(q), _ptr(kv_pages),
                                            _ptr(page_table), _ptr(seq_lens), float(scale), _ptr(out),
                                            _stream(q.device))
    check(st, "mla_decode_paged_noalloc")
    return out


def use_sparse(sparse_prefill: bool, B: int, L: int, N: int,
               min_context: int = SPARSE_PREFILL_MIN_CONTEXT_DEFAULT, batched: bool = False) -> bool:
    """The gate ("Sparse prefill for GLM", section "When it runs"): sparse only when switched
    on, for one sequence, in prefill (L > 1), once the cache holds min_context positions.
    batched=True drops the one-sequence clause (the sparse calls here take B >= 1; the
    pages list batches as a limit of their implementation, "Limits and what to do")."""
    return bool(sparse_prefill) and (B == 1 or (batched and B >= 1)) and L > 1 and N >= min_context


def dsa_prefill(q, kv, q_idx, k_idx, w, topk, *, scale=None, block=4096, query_block=1024,
                sparse_prefill=SPARSE_PREFILL_DEFAULT, min_context=SPARSE_PREFILL_MIN_CONTEXT_DEFAULT,
                batched_sparse=False):
    """One chunk of DSA prefill: indexer top-k, then gated attention.

    q [L,H,576], kv [N,576] (N includes this chunk), q_idx [L,32,128], k_idx [N,128], w [L,32],
    or all with a leading batch dimension B. Returns (out [..,L,H,512], idx [..,L,topk]).
    """
    B = q.shape[0] if q.dim() == 4 else 1
    L, N = q.shape[-3], kv.shape[-2]
    idx = dsa_indexer_topk(q_idx, k_idx, w, topk, block=block)
    if use_sparse(sparse_prefill, B, L, N, min_context, batched=batched_sparse):
        return mla_prefill_sparse(q, kv, idx, scale=scale, query_block=query_block), idx
    # below the gate: the dense path over every visible key under the top-k selection
    return mla_prefill_masked(q, kv, idx, scale=scale), idx


class kernel_trace:
    """Context manager: per-kernel HIP-event timing of every library launch inside the block.

        with kernel_trace() as tr:
            ...
        tr.stats -> {kernel name: (launches, total ms)}
    """

    def __enter__(self):
        lib().dsa_mla_trace_collect(0, None, None, None)   # drop stale records
        self._prev = lib().dsa_mla_trace_enable(1)
        self.stats = {}
        return self

    def __exit__(self, *exc):
        lib().dsa_mla_trace_enable(self._prev)
        n_max = 64
        names = ctypes.create_string_buffer(32 * n_max)
        counts = (ctypes.c_int * n_max)()
        tot = (ctypes.c_double * n_max)()
        n = lib().dsa_mla_trace_collect(n_max, names, counts, tot)
        for j in range(min(n, n_max)):
            nm = names.raw[32 * j:32 * j + 32].split(b"\0", 1)[0].decode()
            self.stats[nm] = (counts[j], tot[j])
        return False


def _event_ms(launch, device, reps):
    """Median over reps of one launch's HIP-event time (one untimed launch first)."""
    ts = []
    for r in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize(device)
        if r:
            ts.append(a.elapsed_time(b))
    return sorted(ts)[len(ts) // 2]


def probe_mfma(grid=1024, iters=4096, reps=3, device="cuda"):
    """Sustained bf16 MFMA rate on register operands and the shader clock it runs at
    (diagnostic: the measured ceiling of the matrix-bound kernels). Returns TFLOP/s
    (median launch), the mean shader clock under the load and cycles per MFMA."""
    dev = torch.device(device)
    cyc = torch.empty(4 * grid, dtype=torch.int64, device=dev)
    wall = torch.empty(4 * grid, dtype=torch.int64, device=dev)
    sink = torch.empty(256 * grid, dtype=torch.float32, device=dev)
    khz = ctypes.c_int(0)

    def launch():
        with _on(dev):
            check(lib().dsa_mla_probe_mfma(grid, iters, _ptr(cyc), _ptr(wall), _ptr(sink), ctypes.byref(khz),
                                           _stream(dev)), "dsa_mla_probe_mfma")

    ms = _event_ms(launch, dev, reps)
    c, w = cyc.double().mean().item(), wall.double().mean().item()
    flop = grid * 4 * iters * 8 * 32768
    return {"tflops": flop / ms / 1e9, "sclk_ghz": c / (w / (khz.value * 1e3)) / 1e9,
            "cycles_per_mfma": c / (iters * 8), "ms": ms,
            "what": f"{grid} workgroups x 4 waves, {iters} rounds of 8 independent 32x32x16 bf16 MFMAs"}


def probe_stream(nbytes=2 << 30, mode="copy", grid=2048, reps=3, device="cuda"):
    """HBM stream rate (diagnostic: the measured ceiling of the bandwidth-bound kernels).
    mode "copy" reads and writes nbytes (2 nbytes moved), "read" reads nbytes."""
    dev = torch.device(device)
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty(nbytes // 4 if mode == "copy" else 256 * grid, dtype=torch.int32, device=dev)
    m = {"copy": 0, "read": 1}[mode]

    def launch():
        with _on(dev):
            check(lib().dsa_mla_probe_stream(m, _ptr(src), _ptr(dst), nbytes, grid, _stream(dev)),
                  "dsa_mla_probe_stream")

    ms = _event_ms(launch, dev, reps)
    moved = nbytes * (2 if m == 0 else 1)
    del src, dst
    return {"GB_s": moved / ms / 1e6, "ms": ms, "what": f"{mode} of {nbytes >> 20} MiB, {grid} workgroups"}
