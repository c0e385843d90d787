"""Build libdsa_mla.so in-tree with hipcc for gfx950.

Usage: python -m dsa_sparse_attention_mla_amd.build   (or __graft_entry__.build()).
Compiles every source under csrc/ to an object, in parallel, then links the
shared library next to this file. Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa_mla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# packed fp32 ops are disabled: the compiler would otherwise form v_pk_*_f32 from scalar code.
# MFMA accumulators are kept in ordinary VGPRs (not AGPRs) unless a source is listed in
# AGPR_FORM: the online-softmax rescale of the output accumulators then needs no
# AGPR<->VGPR copies.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Sources whose MFMA accumulators go to the accumulation registers (AGPRs): kernels that
# run one wave per SIMD and need more than 256 registers per lane.
AGPR_FORM = {"attn_absorbed_dense.hip"}


def flags(src):
    f = list(COMMON)
    if os.path.basename(src) in AGPR_FORM:
        i = f.index("-amdgpu-mfma-vgpr-form")
        del f[i - 1:i + 1]
    return f


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
