"""Helpers for GPU tests: move synth tensors to the device, compare with tolerances."""
import numpy as np
import torch

from synth import to_torch


def dev(t, device="cuda:0"):
    """synth Tensor (or numpy array) -> torch device tensor with the same storage bits."""
    return to_torch(t, device)


def host_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def err_report(got, ref):
    d = np.abs(got - ref)
    return dict(max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                rel=float(d.max() / max(np.abs(ref).max(), 1e-30)) if d.size else 0.0)


def assert_close(got, ref, atol, what="", rel_guard=None):
    """max-abs within atol (the stated tolerance); with rel_guard, also max-abs / max|ref|
    within rel_guard, a regression guard a few bf16 ulps above what the kernels reach,
    so that an error well inside the loose absolute bound still fails."""
    r = err_report(got, ref)
    print(f"[{what}] max_abs={r['max_abs']:.3e} mean_abs={r['mean_abs']:.3e} max_abs/max|ref|={r['rel']:.3e}", flush=True)
    assert r["max_abs"] <= atol, f"{what}: max_abs {r['max_abs']} > {atol}"
    if rel_guard is not None:
        assert r["rel"] <= rel_guard, f"{what}: max_abs/max|ref| {r['rel']} > {rel_guard}"
    return r


def sorted_rows(idx: np.ndarray):
    return [sorted(int(x) for x in r if x >= 0) for r in idx]
