"""MLA prefill and DSA sparse prefill on AMD Instinct MI355X (gfx950).

Thin Python binding over libdsa_mla.so. Every function here only marshals
torch device tensors into the C ABI (pointers, sizes, the current HIP stream,
a workspace buffer) -- all arithmetic runs in the library's HIP kernels.

    mla_prefill_dense(...)    non-absorbed (fp32/bf16) or absorbed (bf16) causal prefill
    dsa_indexer_topk(...)     exact indexer top-k with a running selection
    mla_prefill_sparse(...)   absorbed attention over gathered top-k rows
    mla_prefill_masked(...)   dense absorbed attention under the top-k mask (gated path)
    mla_decode_paged(...)     one decode step over a paged joined cache
    mla_decode_paged_noalloc(...)  the same step without a workspace (fixed device scratch)
    use_sparse(...)           the dense/sparse gate ("Sparse prefill for GLM", "When it runs")
    dsa_prefill(...)          indexer + gated attention for one chunk
    probe_mfma(), probe_stream()  measured matrix and HBM ceilings (diagnostics)
"""
from .api import (  # noqa: F401
    mla_prefill_dense, dsa_indexer_topk, mla_prefill_sparse, mla_prefill_masked, masked_workspace_bytes,
    mla_decode_paged, decode_workspace_bytes, mla_decode_paged_noalloc,
    use_sparse, dsa_prefill,
    SPARSE_PREFILL_DEFAULT, SPARSE_PREFILL_MIN_CONTEXT_DEFAULT, kernel_trace, indexer_workspace_bytes,
    probe_mfma, probe_stream,
)
from ._lib import DsaMlaError, lib, LIB_PATH  # noqa: F401
