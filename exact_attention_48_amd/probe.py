"""ctypes binding of libfa_probe.so: measurement kernels timed beside the library.

fa_probe_dq_atomics issues exactly the fp32 atomic adds that a dQ accumulated
from the dK/dV kernel would need (see csrc/probe_dq_atomics.hip); bench.py times
it against the separate dQ pass.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_probe.so")
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_48_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.fa_probe_dq_atomics.argtypes = [vp, ci, ci, ci, ci, ci, vp]
        lib.fa_probe_dq_atomics.restype = ci
        _lib = lib
    return _lib


def dq_atomics(dq_acc, B: int, H: int, N: int, d: int, causal: int, stream=None) -> None:
    """Add the fused design's dQ blocks (value 1.0 each) into dq_acc, fp32 [B, N, H, d]."""
    ptr = dq_acc.data_ptr() if hasattr(dq_acc, "data_ptr") else dq_acc
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    st = stream if isinstance(stream, int) else stream.cuda_stream
    err = load().fa_probe_dq_atomics(ctypes.c_void_p(ptr), B, H, N, d, int(causal), ctypes.c_void_p(st))
    if err != 0:
        raise RuntimeError(f"fa_probe_dq_atomics: hip error {err}")
