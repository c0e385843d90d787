"""The measurement probes run and report plausible figures; the copy probe moves the
bytes it claims to move."""
import pytest
import torch

import dsa_sparse_attention_mla_amd as dm

pytestmark = pytest.mark.gpu


def test_probe_mfma_rate_and_clock():
    r = dm.probe_mfma(grid=256, iters=256, reps=1)
    # 32 cycles per 32x32x16 bf16 MFMA when eight chains are in flight
    assert 30.0 < r["cycles_per_mfma"] < 40.0, r
    assert 0.5 < r["sclk_ghz"] < 2.6, r
    assert 50.0 < r["tflops"] < 2600.0, r


def test_probe_stream_copy_moves_the_bytes():
    n = 64 << 20
    src = torch.arange(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    st = dm.lib().dsa_mla_probe_stream(0, src.data_ptr(), dst.data_ptr(), n, 512,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    r = dm.probe_stream(256 << 20, mode="read", reps=1)
    assert r["GB_s"] > 100.0, r
