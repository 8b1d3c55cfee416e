"""ctypes binding of libfa.so, with the C ABI's own names (include/fa.h).

Argument marshalling only: PyTorch tensors are passed as device pointers, the
current HIP stream as ``stream``; every step of the computation runs in the
library's kernels. The library must have been built (``python -m
exact_attention_48_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4

FA_EXP_HW = 0
FA_EXP_POLY = 1

FA_BWD_PREPROCESS = 1
FA_BWD_DKDV = 2
FA_BWD_DQ = 4
FA_BWD_ALL = 7

EXPORTED = ("fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_bwd_ex", "fa_bwd_workspace_size", "fa_fwd_fp8", "fa_fwd_fp8_ex",
            "fa_fwd_fp8_blockscale",
            "fa_fwd_split", "fa_fwd_split_ex", "fa_merge", "fa_exp2_eval", "fa_status_string", "fa_version",
            "fa_bwd_noalloc", "fa_bwd_noalloc_max_workspace")


class FaOptions(ctypes.Structure):
    """Mirror of ``fa_fwd_options``."""
    _fields_ = [("exp_mode", ctypes.c_int), ("rescale_tau", ctypes.c_float), ("lpt_order", ctypes.c_int)]


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libfa.so (once). Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_48_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp]
    lib.fa_fwd.restype = ci
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, ctypes.POINTER(FaOptions), vp]
    lib.fa_fwd_ex.restype = ci
    lib.fa_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp, sz, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp, sz, ci, vp]
    lib.fa_bwd_ex.restype = ci
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp]
    lib.fa_bwd_noalloc.restype = ci
    lib.fa_bwd_noalloc_max_workspace.argtypes = []
    lib.fa_bwd_noalloc_max_workspace.restype = sz
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_fwd_fp8_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp,
                                  ctypes.POINTER(FaOptions), vp]
    lib.fa_fwd_fp8_ex.restype = ci
    lib.fa_fwd_fp8_blockscale.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp,
                                          ctypes.POINTER(FaOptions), vp]
    lib.fa_fwd_fp8_blockscale.restype = ci
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.fa_fwd_split.restype = ci
    lib.fa_fwd_split_ex.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, ctypes.POINTER(FaOptions), vp]
    lib.fa_fwd_split_ex.restype = ci
    lib.fa_merge.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, vp]
    lib.fa_merge.restype = ci
    lib.fa_exp2_eval.argtypes = [vp, vp, ctypes.c_int64, ci, vp]
    lib.fa_exp2_eval.restype = ci
    lib.fa_status_string.argtypes = [ci]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (or an int address / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_version() -> str:
    return load().fa_version().decode()


def fa_fwd(q, k, v, o, lse, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int, softmax_scale: float,
           cu_seqlens=None, stream=None, check: bool = True) -> int:
    st = load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(causal),
                       float(softmax_scale), _ptr(cu_seqlens), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd")
    return st


def fa_fwd_ex(q, k, v, o, lse, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int, softmax_scale: float,
              cu_seqlens=None, options: Optional[FaOptions] = None, stream=None, check: bool = True) -> int:
    opt = ctypes.byref(options) if options is not None else None
    st = load().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(causal),
                          float(softmax_scale), _ptr(cu_seqlens), opt, _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_ex")
    return st


def fa_bwd_workspace_size(B: int, Hq: int, Hkv: int, N: int, d: int, causal: int, varlen: int) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, Hkv, N, d, int(causal), int(varlen)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int,
           softmax_scale: float, cu_seqlens=None, workspace=None, workspace_bytes: int = 0, stream=None,
           check: bool = True) -> int:
    st = load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                       B, Hq, Hkv, N, d, int(causal), float(softmax_scale), _ptr(cu_seqlens), _ptr(workspace),
                       int(workspace_bytes), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_bwd")
    return st


def fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int,
              softmax_scale: float, cu_seqlens=None, workspace=None, workspace_bytes: int = 0,
              stages: int = FA_BWD_ALL, stream=None, check: bool = True) -> int:
    st = load().fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), B, Hq, Hkv, N, d, int(causal), float(softmax_scale), _ptr(cu_seqlens),
                          _ptr(workspace), int(workspace_bytes), int(stages), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_bwd_ex")
    return st


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int,
                   softmax_scale: float, cu_seqlens=None, stream=None, check: bool = True) -> int:
    st = load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), B, Hq, Hkv, N, d, int(causal), float(softmax_scale), _ptr(cu_seqlens),
                               _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")
    return st


def fa_bwd_noalloc_max_workspace() -> int:
    return int(load().fa_bwd_noalloc_max_workspace())


def fa_fwd_split(q, k, v, o_part, lse_part, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, causal: int,
                 softmax_scale: float, n_splits: int, stream=None, check: bool = True) -> int:
    st = load().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, Hq, Hkv, Nq, Nk, d,
                             int(causal), float(softmax_scale), int(n_splits), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_split")
    return st


def fa_fwd_split_ex(q, k, v, o_part, lse_part, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, causal: int,
                    softmax_scale: float, n_splits: int, options: Optional[FaOptions] = None, stream=None,
                    check: bool = True) -> int:
    opt = ctypes.byref(options) if options is not None else None
    st = load().fa_fwd_split_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, Hq, Hkv, Nq, Nk, d,
                                int(causal), float(softmax_scale), int(n_splits), opt, _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_split_ex")
    return st


def fa_merge(o_part, lse_part, o, lse, n_parts: int, B: int, H: int, N: int, d: int, stream=None,
             check: bool = True) -> int:
    st = load().fa_merge(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), int(n_parts), B, H, N, d,
                         _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_merge")
    return st


def fa_exp2_eval(x, y, n: int, exp_mode: int, stream=None, check: bool = True) -> int:
    st = load().fa_exp2_eval(_ptr(x), _ptr(y), int(n), int(exp_mode), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_exp2_eval")
    return st


def fa_fwd_fp8(q8, k8, v, q_descale, k_descale, o, lse, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int,
               softmax_scale: float, cu_seqlens=None, stream=None, check: bool = True) -> int:
    st = load().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(o), _ptr(lse), B,
                           Hq, Hkv, N, d, int(causal), float(softmax_scale), _ptr(cu_seqlens), _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return st


def fa_fwd_fp8_ex(q8, k8, v, q_descale, k_descale, o, lse, B: int, Hq: int, Hkv: int, N: int, d: int, causal: int,
                  softmax_scale: float, cu_seqlens=None, options: Optional[FaOptions] = None, stream=None,
                  check: bool = True) -> int:
    opt = ctypes.byref(options) if options is not None else None
    st = load().fa_fwd_fp8_ex(_ptr(q8), _ptr(k8), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(o), _ptr(lse),
                              B, Hq, Hkv, N, d, int(causal), float(softmax_scale), _ptr(cu_seqlens), opt,
                              _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_ex")
    return st


def fa_fwd_fp8_blockscale(q8, k8, v, q_descale, k_descale, o, lse, B: int, Hq: int, Hkv: int, N: int, d: int,
                          causal: int, softmax_scale: float, cu_seqlens=None, options: Optional[FaOptions] = None,
                          stream=None, check: bool = True) -> int:
    opt = ctypes.byref(options) if options is not None else None
    st = load().fa_fwd_fp8_blockscale(_ptr(q8), _ptr(k8), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(o),
                                      _ptr(lse), B, Hq, Hkv, N, d, int(causal), float(softmax_scale),
                                      _ptr(cu_seqlens), opt, _stream(stream))
    if check and st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_blockscale")
    return st
