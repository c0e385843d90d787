#!/usr/bin/env python3
"""Benchmark: DSA sparse MLA prefill at 128K context on one MI355X.

One step = one pass of the sparse-prefill hot path over one chunk: the indexer
(32 heads x 128, weighted ReLU head sum, exact top-2048 over N = 131072 keys)
followed by absorbed attention for 64 heads over each query's 2048 gathered
576-wide latent+rope rows, for a chunk of L = 1024 queries at the end of the
context. Inputs are seeded synthetic data of those shapes, resident in HBM
before timing starts. value = L / step time (prefill tokens per second).

The line also carries:
  roofline      the dominant kernel's achieved rate against the MI355X peak of
                its bound, timed with HIP events on its launch stream;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload on this host (per stage, with the CPU model and BLAS
                library; the masked dense definition on two of the rows), and
                the oracle of the two dense configurations on a few rows each;
  graph_ms_per_step  the same step captured once into a HIP graph and replayed
                (value itself is the eagerly launched step);
  pages_protocol_ms  the step timed as the pages time theirs: the mean of
                three runs after one warm-up run;
  kernels_ms    per-kernel average duration (HIP events);
  other_configs the other configurations, each with its roofline fraction:
                non-absorbed fp32 at L = N = 256 and bf16 at L = N = 4096,
                absorbed bf16 at L = 512 / N = 16384, the indexer alone at
                L = 512 / N = 65536, and a paged decode step.
  measured_ceilings  what this GPU sustains, measured in the same run by the
                library's probes: bf16 MFMA on register operands (with the
                shader clock under that load) and HBM copy / read streams;
                the fractions above are also given against these.

  traffic       HBM bytes per launch of the dominant kernel from rocprofv3's
                FETCH_SIZE / WRITE_SIZE counters, scaled by what the same
                counters read for a plain copy of known size
                (python bench.py --copy-calibration 1024); null once the
                kernel's source differs from the one the counters were taken on.

  dense_baseline the path the sparse call replaces (masked dense attention) on
                the same chunk, with the speed-ups of the sparse path.

Kernel and configuration times are medians of per-launch HIP-event timings
(launches queued back to back).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--no-cpu-baseline]
       python bench.py --sweep        context sweep, sparse vs masked dense
       python bench.py --copy-calibration MIB
       python bench.py --dense-only   the dense configurations alone
       python bench.py --ceilings-only  the measurement probes alone
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

L, N, TOPK, BLOCK, H = 1024, 131072, 2048, 4096, 64
SEED = 1004

# rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) on a 1 GiB device copy read
# 524302 KiB fetched and 1048576 KiB written per dispatch: fetch counts half the
# bytes a copy moves on this chip, write counts all of them.
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
# Counter readings (KiB per dispatch, mean of the 32 launches of this workload in a
# 2-step bench run) and a digest of the kernel sources they were taken on.
COUNTERS = {
    "indexer_score_filter": {"fetch_kib": 165026.3, "write_kib": 40808.1,
                             "sources": ("indexer.hip", "common.h"), "sha256_16": "a94cf04ce43558de"},
    "sparse_attn": {"fetch_kib": 891426.7, "write_kib": 66028.6,
                    "sources": ("attn_absorbed.hip", "common.h"), "sha256_16": "22423f6382a19b7c"},
}
METRIC = "prefill tok/s at 128K ctx (sparse MLA); MFMA util %, HBM GB/s % of peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def indexer_flops(L, N):
    """8192 FLOP (32 heads x 128-dim dot, multiply-add) per visible (query, key) pair."""
    visible = sum(min(N, N - L + i + 1) for i in range(L))
    return 2 * 32 * 128 * visible


def sparse_attn_bytes(L, topk, H):
    """Algorithmic HBM bytes of one sparse attention launch: gathered rows, q, out, idx."""
    return L * topk * 576 * 2 + L * H * 576 * 2 + L * H * 512 * 2 + L * topk * 4


def sparse_attn_flops(L, topk, H):
    return L * topk * H * 2 * (576 + 512)


def traffic_bytes(kernel):
    """HBM bytes per launch from the calibrated counters, or None if the kernel changed since."""
    import hashlib
    c = COUNTERS.get(kernel)
    if c is None:
        return None
    m = hashlib.sha256()
    for f in c["sources"]:
        with open(os.path.join(HERE, "dsa_sparse_attention_mla_amd", "csrc", f), "rb") as fh:
            m.update(fh.read())
    if m.hexdigest()[:16] != c["sha256_16"]:
        return None
    return (c["fetch_kib"] * FETCH_FACTOR + c["write_kib"] * WRITE_FACTOR) * 1024.0


def copy_calibration(mib):
    """A plain device copy of `mib` MiB, three times, for calibrating the byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB three times")


def cpu_baseline(g, sample):
    """The fp64 oracle on `sample` query rows of the same workload, on this host's cores."""
    import numpy as np
    import oracle
    from synth import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rows = np.linspace(0, L - 1, sample).astype(int)
    qf, kf, wf = to_f64(g["q_idx"]), to_f64(g["k_idx"]), to_f64(g["w"])
    q64 = to_f64(g["q"])
    kv64 = to_f64(g["kv"])
    t0 = time.perf_counter()
    s = oracle.indexer_scores(qf, kf, wf, rows=rows)
    t1 = time.perf_counter()
    sel = oracle.topk_full(s, TOPK)
    idx = np.full((L, TOPK), -1, dtype=np.int64)
    idx[rows] = sel
    t2 = time.perf_counter()
    oracle.mla_sparse_gather(q64, kv64, idx, 1.0 / np.sqrt(576.0), rows=rows)
    t3 = time.perf_counter()
    dt = t3 - t0
    # the dense path under the same selection (the definition the gather form equals), on
    # two of the sampled rows: every one of the 131072 keys scored for each head
    mrows = rows[:2]
    t4 = time.perf_counter()
    oracle.mla_masked_dense(q64, kv64, idx, 1.0 / np.sqrt(576.0), rows=mrows)
    t5 = time.perf_counter()
    return {"value": sample / dt, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{sample} of the {L} query rows (evenly spaced) of the same workload: canonical fp64 indexer "
                      f"scores over all {N} keys, full stable-sort top-{TOPK}, fp64 gather attention over {H} heads; "
                      f"{dt:.1f} s",
            "stages_s": {"indexer_scores": t1 - t0, "topk_full_sort": t2 - t1, "sparse_gather_attention": t3 - t2},
            "masked_dense_s_per_row": (t5 - t4) / len(mrows),
            "host": host_info()}


def host_info():
    """CPU model and the BLAS library NumPy uses, for the oracle timings."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: i.get(k) for k in ("internal_api", "version", "num_threads")}
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_dense_stages(rows1=256, rows2=16):
    """The fp64 oracle of the two dense configurations on a few query rows each (the
    last rows, which see the most keys): seconds per row, beside the GPU kernels."""
    import numpy as np
    import oracle
    from synth import gen_absorbed, gen_nonabsorbed, to_f64
    out = {}
    g = gen_nonabsorbed(1001, 4096, 4096, H=16, dtype="bf16", scale=0.5)
    a = {k: to_f64(v) for k, v in g.items()}
    r = np.arange(4096 - rows1, 4096)
    t0 = time.perf_counter()
    oracle.mla_nonabsorbed(a["qn"], a["qr"], a["kn"], a["kr"], a["v"], 1.0 / np.sqrt(192.0), rows=r)
    out["nonabsorbed_bf16_L4096_N4096_H16"] = {"rows": rows1, "s_per_row": (time.perf_counter() - t0) / rows1}
    g = gen_absorbed(1002, 512, 16384, H=64)
    q64, kv64 = to_f64(g["q"]), to_f64(g["kv"])
    r = np.arange(512 - rows2, 512)
    t0 = time.perf_counter()
    oracle.mla_absorbed(q64, kv64, 1.0 / np.sqrt(576.0), rows=r)
    out["absorbed_bf16_L512_N16384_H64"] = {"rows": rows2, "s_per_row": (time.perf_counter() - t0) / rows2}
    return out


def dense_configs(dm, torch, reps=10, ceil=None):
    """Time the dense MLA prefill configurations (not part of the step)."""
    from synth import gen_absorbed, gen_nonabsorbed
    from synth import to_torch as dev
    res = {}

    def entry(ms, fl, peak, measured=None):
        e = {"ms": ms, "tflops": fl / ms / 1e9, "mfma_frac": fl / ms / 1e9 / peak}
        if measured:
            e["frac_of_measured_mfma"] = fl / ms / 1e9 / measured
        return e
    meas = ceil["mfma_bf16"]["tflops"] if ceil else None
    g = gen_nonabsorbed(1000, 256, 256, H=16, dtype="f32")
    t = {k: dev(v)[None] for k, v in g.items()}
    fn = lambda: dm.mla_prefill_dense(t["qn"], t["kn"], q_rope=t["qr"], k_rope=t["kr"], v=t["v"])  # noqa: E731
    ms = _time(fn, torch, reps)
    res["nonabsorbed_fp32_L256_N256_H16"] = dict(entry(ms, 640 * 16 * 256 * 257 // 2, PEAK_FP32_MFMA_TFLOPS),
                                                 peak="fp32 MFMA 157.3 TFLOP/s",
                                                 note="one 64-query tile per workgroup: 64 workgroups, launch-bound")
    g = gen_nonabsorbed(1001, 4096, 4096, H=16, dtype="bf16", scale=0.5)
    t = {k: dev(v)[None] for k, v in g.items()}
    ms = _time(fn, torch, reps)
    res["nonabsorbed_bf16_L4096_N4096_H16"] = entry(ms, 640 * 16 * 4096 * 4097 // 2, PEAK_BF16_TFLOPS, meas)
    g = gen_absorbed(1002, 512, 16384, H=64)
    q, kv = dev(g["q"])[None], dev(g["kv"])[None]
    ms = _time(lambda: dm.mla_prefill_dense(q, kv), torch, reps)
    fl = 2176 * 64 * sum(16384 - 512 + i + 1 for i in range(512))
    res["absorbed_bf16_L512_N16384_H64"] = entry(ms, fl, PEAK_BF16_TFLOPS, meas)
    return res


def indexer_config(dm, torch, Li=512, Ni=65536, reps=10, ceil=None):
    """The indexer alone at L = 512, N = 65536 (top-2048, blocks of 4096): the phase
    (every indexer kernel) and its score kernel, against bf16 MFMA peak."""
    from synth import gen_indexer
    from synth import to_torch as dev
    g = gen_indexer(1003, Li, Ni)
    q_idx, k_idx, w = dev(g["q_idx"]), dev(g["k_idx"]), dev(g["w"])
    ws = torch.empty(dm.indexer_workspace_bytes(Li, Ni, TOPK, BLOCK), dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((Li, TOPK), dtype=torch.int32, device="cuda:0")
    fn = lambda: dm.dsa_indexer_topk(q_idx, k_idx, w, TOPK, block=BLOCK, out=idx, workspace=ws)  # noqa: E731
    ms = _time(fn, torch, reps)
    with dm.kernel_trace() as tr:
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
    kms = {k: tot / max(cnt, 1) for k, (cnt, tot) in tr.stats.items()}
    fl = indexer_flops(Li, Ni)
    t_sc = max(kms.values()) if kms else ms
    sc_name = max(kms, key=kms.get) if kms else None
    e = {"workload": f"indexer, L={Li}, N={Ni}, 32 heads x 128, top-{TOPK}, blocks of {BLOCK}",
         "ms": ms, "tflops": fl / ms / 1e9, "mfma_frac": fl / ms / 1e9 / PEAK_BF16_TFLOPS,
         "score_kernel": sc_name, "score_kernel_ms": t_sc, "score_kernel_mfma_frac": fl / t_sc / 1e9 / PEAK_BF16_TFLOPS,
         "kernels_ms": kms}
    if ceil:
        e["score_kernel_frac_of_measured_mfma"] = fl / t_sc / 1e9 / ceil["mfma_bf16"]["tflops"]
    return e


def measured_ceilings(dm):
    """The library's probes: sustained bf16 MFMA (and the shader clock under it), HBM streams."""
    mf = dm.probe_mfma(grid=1024, iters=4096)
    cp = dm.probe_stream(2 << 30, mode="copy")
    rd = dm.probe_stream(2 << 30, mode="read")
    return {"mfma_bf16": mf, "hbm_copy": cp, "hbm_read": rd,
            "mfma_frac_of_datasheet": mf["tflops"] / PEAK_BF16_TFLOPS,
            "hbm_read_frac_of_datasheet": rd["GB_s"] / PEAK_HBM_GBS}


def decode_config(dm, torch, B=8, n=131072, page_size=64, reps=10):
    """One decode step (L = 1, 64 heads) for B sequences of n keys each, over a paged
    joined cache with shuffled page placement. HBM-bound: the step reads every row once."""
    g = torch.Generator(device="cpu").manual_seed(SEED)
    npg = (n + page_size - 1) // page_size
    pages = torch.randn((B * npg, page_size, 576), generator=g).to(torch.bfloat16).cuda()
    q = torch.randn((B, H, 576), generator=g).to(torch.bfloat16).cuda()
    table = torch.randperm(B * npg, generator=g).to(torch.int32).view(B, npg).cuda()
    lens = torch.full((B,), n, dtype=torch.int32).cuda()
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dm.decode_workspace_bytes(B, H, B * npg, page_size, npg), dtype=torch.uint8, device="cuda")
    ms = _time(lambda: dm.mla_decode_paged(q, pages, table, lens, out=out, workspace=ws), torch, reps)
    by = B * n * 1152 + B * H * 576 * 2 + B * H * 512 * 2 + B * npg * 4
    return {"workload": f"decode step, {B} sequences x {n} keys, {H} heads, pages of {page_size} rows",
            "ms": ms, "GB_s": by / ms / 1e6, "frac_hbm": by / ms / 1e6 / PEAK_HBM_GBS,
            "tflops": B * n * H * 2176 / ms / 1e9}


def sparse_cold(dm, torch, q, kv, idx, out, reps=5):
    """Sparse attention with cold caches: a 512 MB fill (twice the 256 MB last-level cache)
    runs before each timed call, so the gathered rows come from HBM. Median of reps calls."""
    ev = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ts = []
    for r in range(reps + 1):
        ev.fill_(r & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dm.mla_prefill_sparse(q, kv, idx, out=out, query_block=1024)
        b.record()
        torch.cuda.synchronize()
        if r:
            ts.append(a.elapsed_time(b))
    del ev
    ms = sorted(ts)[len(ts) // 2]
    by = sparse_attn_bytes(L, TOPK, H)
    return {"ms": ms, "achieved_GBs": by / (ms * 1e-3) / 1e9, "frac_hbm": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "protocol": f"512 MB fill before each call, median of {reps}"}


def masked_baseline(dm, torch, q, kv, idx, t_sparse_ms, step_ms, reps=3):
    """The path the sparse call replaces, on the same chunk: dense absorbed attention over
    every visible key under the same top-k selection ("Sparse prefill for GLM", "The dense
    mask"). Not part of the step; reported with the sparse speed-ups it implies."""
    ws = torch.empty(dm.masked_workspace_bytes(1, L, N), dtype=torch.uint8, device=q.device)
    out = torch.empty((L, H, 512), dtype=torch.bfloat16, device=q.device)
    ms = _time(lambda: dm.mla_prefill_masked(q, kv, idx, out=out, workspace=ws), torch, reps)
    visible = sum(min(N, N - L + i + 1) for i in range(L))
    fl = 2176 * H * visible
    return {"workload": f"masked dense absorbed attention, L={L}, N={N}, {H} heads, top-{TOPK} mask",
            "ms": ms, "tflops": fl / ms / 1e9, "mfma_frac": fl / ms / 1e9 / PEAK_BF16_TFLOPS,
            "attention_speedup_sparse": ms / t_sparse_ms if t_sparse_ms else None,
            "step_speedup_sparse": (step_ms - t_sparse_ms + ms) / step_ms if t_sparse_ms else None}


def sweep(dm, torch, dev):
    """Chunked-prefill context sweep ("Sparse prefill for GLM", "When it runs" and the
    prompt-length benchmark): for each context N and chunk length L, one prefill step of
    the chunk with the sparse path (indexer + gathered attention) and with the path it
    replaces (indexer + masked dense attention); the crossover places the gate's minimum
    context on this GPU. Inputs: one synthetic draw at the largest sizes, sliced."""
    from synth import gen_dsa_prefill
    Nmax, Lmax = 131072, 1024
    g = gen_dsa_prefill(SEED, Lmax, Nmax, H=H)
    full = {k: dev(g[k]) for k in ("q_idx", "k_idx", "w", "q", "kv")}
    rows = []
    for n in (4096, 8192, 16384, 32768, 65536, 131072):
        for l in (512, 1024):
            q_idx, w, q = full["q_idx"][:l], full["w"][:l], full["q"][:l]
            k_idx, kv = full["k_idx"][:n], full["kv"][:n]
            ws = torch.empty(dm.indexer_workspace_bytes(l, n, TOPK, BLOCK), dtype=torch.uint8, device=q.device)
            mws = torch.empty(dm.masked_workspace_bytes(1, l, n), dtype=torch.uint8, device=q.device)
            idx = torch.empty((l, TOPK), dtype=torch.int32, device=q.device)
            out = torch.empty((l, H, 512), dtype=torch.bfloat16, device=q.device)
            t_idx = _time(lambda: dm.dsa_indexer_topk(q_idx, k_idx, w, TOPK, block=BLOCK, out=idx, workspace=ws),
                          torch, 5)
            t_sp = _time(lambda: dm.mla_prefill_sparse(q, kv, idx, out=out), torch, 5)
            t_md = _time(lambda: dm.mla_prefill_masked(q, kv, idx, out=out, workspace=mws), torch, 3)
            row = {"N": n, "L": l, "indexer_ms": t_idx, "sparse_attn_ms": t_sp, "masked_dense_attn_ms": t_md,
                   "sparse_tok_s": l / ((t_idx + t_sp) * 1e-3), "dense_tok_s": l / ((t_idx + t_md) * 1e-3),
                   "speedup": (t_idx + t_md) / (t_idx + t_sp), "gate_says_sparse": bool(dm.use_sparse(True, 1, l, n))}
            log(f"sweep N={n} L={l}: sparse {row['sparse_tok_s']:.0f} tok/s, dense {row['dense_tok_s']:.0f} tok/s, "
                f"x{row['speedup']:.2f}")
            rows.append(row)
    wins = [r["N"] for r in rows if r["speedup"] > 1.0]
    return {"sweep": rows, "smallest_context_where_sparse_wins": min(wins) if wins else None,
            "gate_min_context": 16384}


def _time(fn, torch, reps):
    """Median over reps of one call's HIP-event time. The calls are queued back to back
    (no synchronisation between them), so each event pair brackets the call's own GPU
    work rather than the host's launch latency. Untimed calls come first, for at least
    30 ms of GPU time: a configuration's first calls after other work run up to 15%
    slower until the GPU settles (measured on the 0.1 ms non-absorbed configuration)."""
    t0 = time.perf_counter()
    for i in range(400):
        fn()
        if i >= 4 and i % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > 0.03:
                break
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=512)
    ap.add_argument("--sweep", action="store_true",
                    help="only run the context sweep (sparse vs masked dense, N = 4K..128K, L = 512/1024)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="only run the measurement probes (MFMA, HBM copy / read) and print them")
    ap.add_argument("--dense-only", action="store_true",
                    help="only time the dense MLA configurations (fp32 and bf16 non-absorbed, absorbed; for counter runs) and print them")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(query sharding needs no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    import dsa_sparse_attention_mla_amd as dm

    if args.dense_only:
        print(json.dumps(dense_configs(dm, torch)), flush=True)
        return
    if args.ceilings_only:
        print(json.dumps(measured_ceilings(dm)), flush=True)
        return
    from synth import gen_dsa_prefill
    from synth import to_torch as dev

    if args.sweep:
        print(json.dumps(sweep(dm, torch, dev)), flush=True)
        return

    log("bench: generating inputs")
    g = gen_dsa_prefill(SEED, L, N, H=H)
    q_idx, k_idx, w, q, kv = (dev(g[k]) for k in ("q_idx", "k_idx", "w", "q", "kv"))
    ws = torch.empty(dm.indexer_workspace_bytes(L, N, TOPK, BLOCK), dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((L, TOPK), dtype=torch.int32, device="cuda:0")
    out = torch.empty((L, H, 512), dtype=torch.bfloat16, device="cuda:0")
    assert dm.use_sparse(True, 1, L, N)

    def step():
        dm.dsa_indexer_topk(q_idx, k_idx, w, TOPK, block=BLOCK, out=idx, workspace=ws)
        dm.mla_prefill_sparse(q, kv, idx, out=out, query_block=1024)

    log("bench: warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: timed steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    # the pages' own protocol: the mean of three runs after one warm-up run
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    pages_protocol_ms = (time.perf_counter() - t0) * 1e3 / 3
    step_median_ms = _time(step, torch, args.steps)

    # the same step captured once into a HIP graph and replayed (no per-launch host work)
    log("bench: graph replay")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    del graph

    log("bench: per-kernel event timing")
    per_kernel = {}
    for _ in range(args.steps):
        with dm.kernel_trace() as tr:
            step()
            torch.cuda.synchronize()
        for k, (cnt, tot) in tr.stats.items():
            per_kernel.setdefault(k, []).append(tot / max(cnt, 1))
    kernels_ms = {k: sorted(v)[len(v) // 2] for k, v in per_kernel.items()}   # median over steps
    t_idx = kernels_ms.get("indexer_score_filter", 0.0)
    t_att = kernels_ms.get("sparse_attn", 0.0)
    log("bench: measured ceilings")
    ceil = measured_ceilings(dm)
    if t_idx >= t_att:
        fl = indexer_flops(L, N)
        ach = fl / (t_idx * 1e-3) / 1e12
        roof = {"kernel": "indexer_score_filter", "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic_bytes("indexer_score_filter"),
                "per_launch": f"{fl:.4e} FLOP (8192 per visible query-key pair)", "ms": t_idx,
                "frac_of_measured": ach / ceil["mfma_bf16"]["tflops"]}
    else:
        by = sparse_attn_bytes(L, TOPK, H)
        ach = by / (t_att * 1e-3) / 1e9
        roof = {"kernel": "sparse_attn", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": traffic_bytes("sparse_attn"),
                "per_launch": f"{by:.4e} B (gathered rows, q, out, idx)", "ms": t_att,
                "frac_of_measured": ach / ceil["hbm_read"]["GB_s"]}

    other = None
    baseline = None
    cold = None
    if not args.no_other_configs:
        log("bench: sparse attention, cold caches")
        cold = sparse_cold(dm, torch, q, kv, idx, out)
        log("bench: dense configurations")
        other = dense_configs(dm, torch, ceil=ceil)
        log("bench: indexer alone (L=512, N=65536)")
        other["indexer_L512_N65536"] = indexer_config(dm, torch, ceil=ceil)
        log("bench: masked dense baseline")
        baseline = masked_baseline(dm, torch, q, kv, idx, t_att, ms_per_step)
        log("bench: paged decode")
        other["paged_decode_B8_N131072_H64"] = decode_config(dm, torch)
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(g, args.cpu_sample)
        cpu["dense_configs"] = cpu_dense_stages()

    line = {
        "metric": METRIC, "value": L / (ms_per_step * 1e-3), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "step_median_ms": step_median_ms,
        "graph_ms_per_step": graph_ms_per_step, "graph_tok_s": L / (graph_ms_per_step * 1e-3),
        "pages_protocol_ms": pages_protocol_ms,
        "config": {"workload": "DSA sparse MLA prefill, one 1024-query chunk at the end of a 131072-position "
                               "context: indexer 32 heads x 128 (top-2048, blocks of 4096) + absorbed attention "
                               "64 heads over gathered 576-wide latent+rope rows (value = first 512)",
                   "L": L, "N": N, "topk": TOPK, "heads": H, "indexer_heads": 32, "block": BLOCK,
                   "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "kernels_ms": kernels_ms,
        "phases_ms": {"indexer_total": sum(v for k, v in kernels_ms.items() if k.startswith(("indexer", "key_norm", "query_eps"))),
                      "sparse_attn": t_att},
        "sparse_attn_roofline": {"effective_GBs_at_algorithmic_bytes": sparse_attn_bytes(L, TOPK, H) / (t_att * 1e-3) / 1e9 if t_att else None,
                                 "effective_frac_hbm": sparse_attn_bytes(L, TOPK, H) / (t_att * 1e-3) / 1e9 / PEAK_HBM_GBS if t_att else None,
                                 "algorithmic_bytes": sparse_attn_bytes(L, TOPK, H),
                                 "counter_bytes": traffic_bytes("sparse_attn"),
                                 "note": "algorithmic bytes count every gathered row once per query; rows shared by "
                                         "queries of the chunk are served from the 256 MB last-level cache, so this "
                                         "is an effective rate, not DRAM bandwidth (counter_bytes: HBM bytes read "
                                         "and written, from rocprofv3, or null if the kernel changed since)",
                                 "tflops": sparse_attn_flops(L, TOPK, H) / (t_att * 1e-3) / 1e12 if t_att else None,
                                 "caches": "warm (the bench step's own)", "cold": cold},
        "other_configs": other,
        "measured_ceilings": ceil,
        "dense_baseline": baseline,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
