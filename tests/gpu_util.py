"""Helpers for GPU tests: move synth tensors to the device, compare with tolerances."""
import numpy as np
import torch

from synth import Tensor


def dev(t, device="cuda:0"):
    """synth Tensor (or numpy array) -> torch device tensor with the same storage bits."""
    if isinstance(t, Tensor):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    return torch.from_numpy(np.ascontiguousarray(t)).to(device)


def host_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def err_report(got, ref):
    d = np.abs(got - ref)
    return dict(max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                rel=float(d.max() / max(np.abs(ref).max(), 1e-30)) if d.size else 0.0)


def assert_close(got, ref, atol, what=""):
    r = err_report(got, ref)
    print(f"[{what}] max_abs={r['max_abs']:.3e} mean_abs={r['mean_abs']:.3e} max_abs/max|ref|={r['rel']:.3e}", flush=True)
    assert r["max_abs"] <= atol, f"{what}: max_abs {r['max_abs']} > {atol}"
    return r


def sorted_rows(idx: np.ndarray):
    return [sorted(int(x) for x in r if x >= 0) for r in idx]
