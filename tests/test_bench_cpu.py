"""Host-side checks of bench.py that need no GPU."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(HERE, "..", "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)



def _bench():
    sys.path.insert(0, os.path.join(HERE, ".."))
    import bench
    return bench


def test_indexer_flops_counts_visible_pairs():
    """8192 FLOP (32 heads x 128 dims x multiply-add) per (query, key) pair the causal
    mask leaves visible: brute force on small shapes, the closed form at the workloads."""
    b = _bench()
    for L, N in [(1, 1), (3, 5), (4, 4), (7, 100)]:
        pairs = sum(1 for i in range(L) for n in range(N) if n <= N - L + i)
        assert b.indexer_flops(L, N) == 8192 * pairs
    for L, N in [(1024, 131072), (512, 65536)]:
        assert b.indexer_flops(L, N) == 8192 * (L * (N - L + 1) + L * (L - 1) // 2)
    assert abs(b.indexer_flops(1024, 131072) - 1.0952e12) < 1e8


def test_sparse_attention_algorithmic_bytes_and_flops():
    """Gathered 576-wide bf16 rows, the bf16 queries and outputs, the int32 index lists;
    (576 + 512) multiply-adds per selected key and head."""
    b = _bench()
    L, k, H = 1024, 2048, 64
    assert b.sparse_attn_bytes(L, k, H) == L * k * 1152 + L * H * 1152 + L * H * 1024 + L * k * 4
    assert abs(b.sparse_attn_bytes(L, k, H) - 2.567e9) < 1e6
    assert b.sparse_attn_flops(L, k, H) == 2 * L * k * H * (576 + 512)


def test_counter_traffic_is_null_once_the_kernel_changed(monkeypatch):
    b = _bench()
    for name, c in b.COUNTERS.items():
        t = b.traffic_bytes(name)
        assert t is None or t == (c["fetch_kib"] * b.FETCH_FACTOR + c["write_kib"] * b.WRITE_FACTOR) * 1024.0
        monkeypatch.setitem(b.COUNTERS, name, dict(c, sha256_16="0" * 16))
        assert b.traffic_bytes(name) is None
    assert b.traffic_bytes("no such kernel") is None
