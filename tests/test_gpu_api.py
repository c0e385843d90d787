"""GPU: the Python binding refuses caller buffers of the wrong shape, dtype or device
before anything is launched (a short buffer would otherwise be written past its end)."""
import pytest
import torch

import dsa_sparse_attention_mla_amd as dm

pytestmark = pytest.mark.gpu


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")


def test_bad_out_buffers_rejected_before_launch():
    L, N, H, topk = 4, 64, 16, 8
    q, kv = _bf(L, H, 576), _bf(N, 576)
    idx = torch.zeros((L, topk), dtype=torch.int32, device="cuda:0")
    sentinel = torch.full((L, H, 511), 3.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        dm.mla_prefill_sparse(q, kv, idx, out=sentinel)                      # short last dim
    with pytest.raises(TypeError):
        dm.mla_prefill_sparse(q, kv, idx, out=torch.zeros((L, H, 512), device="cuda:0"))  # fp32
    with pytest.raises(ValueError):
        dm.mla_prefill_masked(q, kv, idx, out=_bf(L - 1, H, 512))
    with pytest.raises(ValueError):
        dm.mla_prefill_dense(q[None], kv[None], out=_bf(1, L, H, 256))
    qi, ki = _bf(L, 32, 128), _bf(N, 128)
    w = torch.zeros((L, 32), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        dm.dsa_indexer_topk(qi, ki, w, topk, out=torch.zeros((L, topk - 1), dtype=torch.int32, device="cuda:0"))
    with pytest.raises(TypeError):
        dm.dsa_indexer_topk(qi, ki, w, topk, out=torch.zeros((L, topk), dtype=torch.int64, device="cuda:0"))
    with pytest.raises(ValueError):
        dm.dsa_indexer_topk(qi, ki, w, topk, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(TypeError):
        dm.dsa_indexer_topk(qi, ki, w, topk, workspace=torch.zeros(1 << 20, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(ValueError):
        dm.mla_prefill_sparse(q, kv.cpu(), idx)                              # input on another device
    torch.cuda.synchronize()
    assert torch.all(sentinel == 3.0)                                        # nothing was written
