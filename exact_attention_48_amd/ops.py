"""Tensor-level helpers over the C ABI: allocate outputs with PyTorch, call capi.

Tensors are bf16, contiguous, on the GPU, in the layouts of include/fa.h:
uniform Q/O [B, N, Hq, d], K/V [B, N, Hkv, d], LSE [B, Hq, N]; packed
Q/O [T, Hq, d], K/V [T, Hkv, d], LSE [Hq, T] with int32 ``cu_seqlens``.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import capi


def _check(name: str, t: torch.Tensor, dtype=torch.bfloat16):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(q: torch.Tensor, k: torch.Tensor, cu_seqlens: Optional[torch.Tensor], max_seqlen: Optional[int]):
    """(B, N, Hq, Hkv, d) from Q and K, checking that they agree."""
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("uniform batches use [B, N, H, d] tensors")
        B, N, Hq, d = q.shape
        if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
            raise ValueError(f"K shape {tuple(k.shape)} does not match Q {tuple(q.shape)}")
        return B, N, Hq, k.shape[2], d
    _check("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 prefix sums")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed batches use [T, H, d] tensors")
    if k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError(f"K shape {tuple(k.shape)} does not match Q {tuple(q.shape)} (token count T and d)")
    if max_seqlen is None:
        raise ValueError("packed batches need max_seqlen (the maximum sequence length)")
    B = cu_seqlens.numel() - 1
    return B, int(max_seqlen), q.shape[1], k.shape[1], q.shape[2]


def _same_shape(name: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _lse_shape(q: torch.Tensor, B: int, N: int, Hq: int, packed: bool):
    return (Hq, q.shape[0]) if packed else (B, Hq, N)


def forward(q, k, v, causal: bool, scale: Optional[float] = None, cu_seqlens=None, max_seqlen=None,
            options: Optional[capi.FaOptions] = None, stream=None, out=None, lse=None):
    """Returns (O, LSE). ``out``/``lse`` may be preallocated."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t)
    B, N, Hq, Hkv, d = _dims(q, k, cu_seqlens, max_seqlen)
    _same_shape("v", v, k.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lse_shape = _lse_shape(q, B, N, Hq, cu_seqlens is not None)
    if out is not None:
        _check("out", out)
        _same_shape("out", out, q.shape)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    else:
        _check("lse", lse, torch.float32)
        _same_shape("lse", lse, lse_shape)
    capi.fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), scale, cu_seqlens, options, stream)
    return o, lse


def backward(q, k, v, o, lse, do, causal: bool, scale: Optional[float] = None, cu_seqlens=None,
             max_seqlen=None, stream=None, workspace=None, dq=None, dk=None, dv=None):
    """Returns (dQ, dK, dV). ``dq``/``dk``/``dv`` may be preallocated."""
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(n, t)
    _check("lse", lse, torch.float32)
    B, N, Hq, Hkv, d = _dims(q, k, cu_seqlens, max_seqlen)
    _same_shape("v", v, k.shape)
    _same_shape("o", o, q.shape)
    _same_shape("do", do, q.shape)
    _same_shape("lse", lse, _lse_shape(q, B, N, Hq, cu_seqlens is not None))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _check(name, t)
            _same_shape(name, t, like.shape)
        outs.append(t)
    dq, dk, dv = outs
    nbytes = capi.fa_bwd_workspace_size(B, Hq, Hkv, N, d, int(causal), int(cu_seqlens is not None))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _check("workspace", workspace, torch.uint8)
    capi.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, int(causal), scale, cu_seqlens,
                workspace, workspace.numel(), stream)
    return dq, dk, dv


def forward_split(q, k, v, causal: bool, n_splits: int, scale: Optional[float] = None, stream=None,
                  o_part=None, lse_part=None, options: Optional[capi.FaOptions] = None):
    """Split-KV partial results of uniform batches: Q [B, Nq, Hq, d], K/V [B, Nk, Hkv, d].

    Returns (O_part fp32 [n, B, Nq, Hq, d], LSE_part fp32 [n, B, Hq, Nq]).
    """
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("split-KV takes uniform [B, N, H, d] tensors with V shaped like K")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("K/V shape does not match Q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o_part is None:
        o_part = torch.empty((n_splits, B, Nq, Hq, d), dtype=torch.float32, device=q.device)
    else:
        _check("o_part", o_part, torch.float32)
        _same_shape("o_part", o_part, (n_splits, B, Nq, Hq, d))
    if lse_part is None:
        lse_part = torch.empty((n_splits, B, Hq, Nq), dtype=torch.float32, device=q.device)
    else:
        _check("lse_part", lse_part, torch.float32)
        _same_shape("lse_part", lse_part, (n_splits, B, Hq, Nq))
    capi.fa_fwd_split_ex(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, int(causal), scale, n_splits, options,
                         stream)
    return o_part, lse_part


def merge(o_part, lse_part, stream=None, out=None, lse=None):
    """Merge partial results O_part [n, B, N, H, d], LSE_part [n, B, H, N] (fp32) -> (O bf16, LSE fp32)."""
    _check("o_part", o_part, torch.float32)
    _check("lse_part", lse_part, torch.float32)
    if o_part.dim() != 5 or lse_part.dim() != 4:
        raise ValueError("partials are O [n, B, N, H, d] and LSE [n, B, H, N]")
    n, B, N, H, d = o_part.shape
    if tuple(lse_part.shape) != (n, B, H, N):
        raise ValueError("LSE partials do not match the O partials")
    if out is not None:
        _check("out", out)
        _same_shape("out", out, (B, N, H, d))
    o = out if out is not None else torch.empty((B, N, H, d), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_part.device)
    else:
        _check("lse", lse, torch.float32)
        _same_shape("lse", lse, (B, H, N))
    capi.fa_merge(o_part, lse_part, o, lse, n, B, H, N, d, stream)
    return o, lse


def forward_fp8(q8, k8, v, q_descale, k_descale, causal: bool, scale: Optional[float] = None, cu_seqlens=None,
                max_seqlen=None, stream=None, options: Optional[capi.FaOptions] = None):
    """8-bit Q/K forward: q8/k8 uint8 E4M3 codes in the Q/K layouts, v bf16, fp32 descales
    [B, Hq] and [B, Hkv] (per sequence and head, fa_fwd_fp8_ex) or [B, Hq, nb] and [B, Hkv, nb]
    (per 64-token block, nb = ceil(N / 64), fa_fwd_fp8_blockscale). Returns (O bf16, LSE fp32)."""
    _check("q8", q8, torch.uint8)
    _check("k8", k8, torch.uint8)
    _check("v", v)
    _check("q_descale", q_descale, torch.float32)
    _check("k_descale", k_descale, torch.float32)
    B, N, Hq, Hkv, d = _dims(q8, k8, cu_seqlens, max_seqlen)
    if v.shape != k8.shape:
        raise ValueError(f"v has shape {tuple(v.shape)}, expected {tuple(k8.shape)}")
    blocks = q_descale.dim() == 3
    nb = (N + 63) // 64
    _same_shape("q_descale", q_descale, (B, Hq, nb) if blocks else (B, Hq))
    _same_shape("k_descale", k_descale, (B, Hkv, nb) if blocks else (B, Hkv))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse_shape = (B, Hq, N) if cu_seqlens is None else (Hq, q8.shape[0])
    lse = torch.empty(lse_shape, dtype=torch.float32, device=q8.device)
    fn = capi.fa_fwd_fp8_blockscale if blocks else capi.fa_fwd_fp8_ex
    fn(q8, k8, v, q_descale, k_descale, o, lse, B, Hq, Hkv, N, d, int(causal), scale, cu_seqlens, options, stream)
    return o, lse
