"""Shared helpers for the GPU parity tests: inputs to the device, oracle comparisons."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from exact_attention_48_amd import capi, inputs as I, ops

# Tolerances against the float64 oracle fed the same bf16 inputs.
O_MAX_ABS = 1e-2
LSE_MAX_ABS = 1e-3
GRAD_REL_FRO = 2e-2


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp32 device tensor -> float64 numpy (exact)."""
    if t.dtype == torch.bfloat16:
        return I.bf16_bits_to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f64(bits)


def gpu_forward(x: I.Inputs, options=None):
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    cu = torch.from_numpy(x.cu_seqlens).to("cuda:0") if x.cu_seqlens is not None else None
    o, lse = ops.forward(q, k, v, x.causal, x.scale, cu, x.N if cu is not None else None, options)
    torch.cuda.synchronize()
    return q, k, v, cu, o, lse


def oracle_forward(x: I.Inputs, rows=None):
    return oracle.attention_forward(f64(x.q), f64(x.k), f64(x.v), x.scale, x.causal, x.cu_seqlens, rows=rows)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits): 2^(floor(log2 |x|) - 7)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def o_bound(o_ref: np.ndarray) -> np.ndarray:
    """The O gate per element: 1e-2, or one bf16 ulp of the exact value where that is
    larger (|O| >= 2). O is stored as bf16, so above |O| = 2 rounding alone can leave
    an error beyond 1e-2 (half an ulp is 0.0078 at |O| in [2, 4), 0.0156 in [4, 8))."""
    return np.maximum(O_MAX_ABS, bf16_ulp(o_ref))


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    """Max-abs errors on the rows the oracle computed (others are NaN in the reference)."""
    o = host_f64(o_gpu)
    lse = host_f64(lse_gpu)
    mo = ~np.isnan(o_ref)
    ml = ~np.isnan(lse_ref)
    assert mo.any() and ml.any()
    assert np.all(np.isfinite(o[mo])) and np.all(np.isfinite(lse[ml])), f"{label}: non-finite output"
    err = np.abs(o[mo] - o_ref[mo])
    eo = float(np.max(err))
    el = float(np.max(np.abs(lse[ml] - lse_ref[ml])))
    worst = float(np.max(err / o_bound(o_ref[mo])))
    assert worst <= 1.0, (f"{label}: O error {eo:.3e} max-abs, {worst:.3f} of the bound "
                          f"(1e-2, or one bf16 ulp where |O| >= 2)")
    assert el <= LSE_MAX_ABS, f"{label}: LSE max-abs error {el:.3e} > {LSE_MAX_ABS}"
    return eo, el


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))




def block_rows(n_first=64, n_last=64, block=32):
    """Row selector for full-size sequences: the first and the last row of every
    32-row block (the rows of one MFMA query block; every wave of every query
    tile holds whole blocks), plus the first and last rows of the sequence."""
    def sel(s, L):
        r = np.arange(L, dtype=np.int64)
        keep = (r % block == 0) | (r % block == block - 1) | (r < n_first) | (r >= L - n_last)
        return r[keep]
    return sel


def wave_coverage(rows: np.ndarray, L: int, tile: int = 256, wave_rows: int = 32) -> np.ndarray:
    """Compared rows per (query tile, wave slot) for `wave_rows`-row waves of `tile`-row
    workgroups; asserts that every slot holding rows of the sequence has at least two."""
    n_t = (L + tile - 1) // tile
    counts = np.zeros((n_t, tile // wave_rows), dtype=np.int64)
    np.add.at(counts, (rows // tile, (rows % tile) // wave_rows), 1)
    starts = np.arange(n_t)[:, None] * tile + np.arange(tile // wave_rows)[None, :] * wave_rows
    live = starts < L
    assert np.all(counts[live] >= min(2, wave_rows)), "a wave slot of some query tile has no compared row"
    return counts


def poisoned(shape, dtype, guard: int = 4096):
    """A NaN-filled device buffer with `guard` extra NaN elements after the view."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), float("nan"), dtype=dtype, device="cuda:0")
    return buf[:n].view(shape), buf


def assert_fully_written(view: torch.Tensor, buf: torch.Tensor, label: str):
    n = view.numel()
    assert not torch.isnan(view).any(), f"{label}: some element was not written"
    assert torch.isnan(buf[n:]).all(), f"{label}: write past the end"
