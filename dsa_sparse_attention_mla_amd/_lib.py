"""ctypes loader for libdsa_mla.so (the C ABI declared in include/dsa_mla.h).

Loading fails loudly when the library has not been built: there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_mla.so")

OK, INVALID_ARG, UNSUPPORTED, ARCH, WORKSPACE, HIP = range(6)
MODE_NONABSORBED, MODE_ABSORBED = 0, 1
F32, BF16 = 0, 1

# every exported entry point: name -> (restype, argtypes)
_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
SIGNATURES = {
    "mla_prefill_dense": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _f, _i, _p, _sz, _p]),
    "dsa_indexer_topk": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _i, _i, _p, _p, _p, _sz, _p]),
    "mla_prefill_sparse": (_i, [_i, _i, _i, _i, _p, _p, _p, _i, _f, _i, _p, _p, _sz, _p]),
    "mla_prefill_masked": (_i, [_i, _i, _i, _i, _p, _p, _p, _i, _f, _p, _p, _sz, _p]),
    "mla_decode_paged": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _f, _p, _p, _sz, _p]),
    "mla_decode_paged_noalloc": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _f, _p, _p]),
    "mla_decode_paged_noalloc_capacity": (ctypes.c_size_t, []),
    "dsa_mla_trace_enable": (_i, [_i]),
    "dsa_mla_trace_collect": (_i, [_i, ctypes.c_char_p, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]),
    "dsa_mla_probe_mfma": (_i, [_i, _i, _p, _p, _p, ctypes.POINTER(ctypes.c_int), _p]),
    "dsa_mla_probe_stream": (_i, [_i, _p, _p, ctypes.c_size_t, _i, _p]),
    "dsa_mla_status_string": (ctypes.c_char_p, [_i]),
    "dsa_mla_abi_version": (_i, []),
}

_lib = None


class DsaMlaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dsa_sparse_attention_mla_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().dsa_mla_status_string(status).decode()


def check(status: int, call: str) -> None:
    if status != OK:
        raise DsaMlaError(status, call)
