"""The DSA prefill step (indexer, then sparse attention) captured into a HIP graph:
every replay reproduces the eager result bit for bit. The library launches kernels
only (no allocation, no memset, no host synchronisation), so it can be captured when
the caller supplies the workspace and outputs; eager work runs between the replays."""
import pytest
import torch

import dsa_sparse_attention_mla_amd as dm
from synth import gen_dsa_prefill
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L,N", [(256, 32768), (96, 5000)])
def test_dsa_step_replays_as_hip_graph(L, N):
    topk = 2048
    g = gen_dsa_prefill(1050 + L, L, N, H=64)
    t = {k: dev(v) for k, v in g.items()}
    ws = torch.empty(dm.indexer_workspace_bytes(L, N, topk), dtype=torch.uint8, device="cuda")
    idx = torch.empty((L, topk), dtype=torch.int32, device="cuda")
    out = torch.empty((L, 64, 512), dtype=torch.bfloat16, device="cuda")

    def step():
        dm.dsa_indexer_topk(t["q_idx"], t["k_idx"], t["w"], topk, out=idx, workspace=ws)
        dm.mla_prefill_sparse(t["q"], t["kv"], idx, out=out)

    step()
    torch.cuda.synchronize()
    idx_ref, out_ref = idx.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"replay {r}: index sets differ"
        assert torch.equal(out, out_ref), f"replay {r}: attention output differs"


def test_noalloc_decode_replays_as_hip_graph():
    """The decode entry point that allocates nothing is what a caller under graph capture
    uses: a captured step replays to the eager result, with eager decode calls (the
    workspace form and the scratch form on other inputs) run between the replays."""
    import numpy as np
    rng = np.random.default_rng(1060)
    B, H, ps, n = 4, 64, 64, 20000
    npg = (n + ps - 1) // ps
    pages = torch.randn((B * npg + 3, ps, 576), generator=torch.Generator().manual_seed(1061)).to(torch.bfloat16).cuda()
    q = torch.randn((B, H, 576), generator=torch.Generator().manual_seed(1062)).to(torch.bfloat16).cuda()
    table = torch.from_numpy(rng.permutation(B * npg + 3)[: B * npg].astype(np.int32).reshape(B, npg)).cuda()
    lens = torch.tensor([n, 1, 12345, 64], dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    dm.mla_decode_paged_noalloc(q, pages, table, lens, out=out)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dm.mla_decode_paged_noalloc(q, pages, table, lens, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dm.mla_decode_paged_noalloc(q, pages, table, lens, out=out)
    other = torch.empty_like(out)
    for r in range(3):
        out.zero_()
        dm.mla_decode_paged(q[:2], pages, table[:2], lens[:2].flip(0).contiguous())
        dm.mla_decode_paged_noalloc(q[1:], pages, table[1:], lens[1:], out=other[1:])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs"
