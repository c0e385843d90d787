"""CPU oracle for MLA prefill and DSA sparse prefill -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of the entry module and the CPU-baseline leg of
the bench may import or run anything in this package. The product path (the
HIP library and its Python binding) never calls it, and this package imports
nothing from the product path.

Everything here is plain NumPy in float64 (plus pure-Python brute force for
tiny inputs): naive full softmax attention, the canonical indexer score, a full
stable-sort top-k and the running (blocked) top-k written out from its
definition. Sources, cited by page and section:

* Fornax part 5, "Apple M3 vs M5 kernels", section "What the kernel has to
  compute" (the two score contractions with the rope key shared by all heads,
  softmax, then the value product) -> ``attention.mla_nonabsorbed``.
* mlx-lm PR 1997 summary, "Sparse prefill for GLM": section "Sparse attention"
  (joined 576-wide latent+rope row, gather of the chosen rows, absorbed
  attention) -> ``attention.mla_absorbed`` / ``attention.mla_sparse_gather``;
  section "The dense mask" -> ``attention.mla_masked_dense``; section "Blocked
  top-k" -> ``indexer.topk_blocked``; section "When it runs" -> ``gate`` and
  the decode step ``attention.mla_decode_paged``.
* Fornax part 5, section "Paged KV: alignment follows the tile" (rows addressed
  one at a time through the page table) -> ``attention.paged_rows``.

Every function has at least one pin in tests/test_oracle_*.py that does not go
through the function's own formula (brute force, closed forms, identities
with library routines, invariants).
"""
from .attention import (  # noqa: F401
    visible_mask, mla_nonabsorbed, mla_absorbed, mla_masked_dense, mla_sparse_gather, paged_rows,
    mla_decode_paged,
)
from .indexer import indexer_scores, topk_full, topk_blocked, exact_dot_flags  # noqa: F401
from .gate import use_sparse, dsa_prefill  # noqa: F401
