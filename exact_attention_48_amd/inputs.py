"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the benchmark and the CPU reference: it
draws random numbers and rounds them to bfloat16, and it holds none of the
attention arithmetic.

Recipe (the same for every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * for packed variable-length batches the sequence lengths are drawn first,
    ``rng.integers(lo, hi, endpoint=True, size=n_seqs)``, and ``cu_seqlens`` is
    ``[0, cumsum(lengths)]`` as int32;
  * then ``rng.standard_normal(shape, dtype=float32)`` for Q, K, V and (for the
    backward workload) dO, in that order;
  * every float32 draw is rounded to bfloat16 with round-to-nearest-even.

Tensor layouts ("BSHD", contiguous): Q/O/dO ``[B, N, Hq, d]``, K/V
``[B, N, Hkv, d]``; packed: Q ``[T, Hq, d]``, K/V ``[T, Hkv, d]`` with
``T = cu_seqlens[-1]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# bfloat16 <-> float32 bit conversions (round-to-nearest-even)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, returning the uint16 bit patterns.

    Round-to-nearest, ties to even, on the raw IEEE-754 bits; NaN stays a
    quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# --------------------------------------------------------------------------
# OCP E4M3 encoding of inputs (round to nearest, ties to even, saturating)
# --------------------------------------------------------------------------

def _e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by code 0x00..0x7E."""
    m = np.arange(8, dtype=np.float64)
    vals = [m / 8.0 * 2.0 ** -6]
    for e in range(1, 16):
        vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.concatenate(vals)[:0x7F]


_E4M3 = _e4m3_magnitudes()


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to OCP E4M3 (nearest, ties to the even code; magnitudes
    above 448 saturate to 448), returning uint8 codes. NaN maps to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), _E4M3[-1])
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _E4M3[lo], _E4M3[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x) & (code != 0), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd", "bwd", "split" or "fp8"
    Hq: int
    Hkv: int
    d: int
    causal: bool
    seed: int
    B: int = 1           # batch size (uniform) or number of sequences (packed)
    N: int = 0           # sequence length (uniform); max length (packed, set on draw)
    varlen: bool = False
    len_lo: int = 0      # packed: inclusive length range of the uniform draw
    len_hi: int = 0
    Nk: int = 0          # split-KV: keys per sequence (N is then the number of queries)
    n_splits: int = 0    # split-KV: key chunks

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to float32 (the value passed to the kernels)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


# Workloads (names say what they are): the five measured configurations, then
# the packed GQA backward and two long-context runs.
WORKLOADS = {
    "fwd_b1_h2_n256_d64": Workload(
        "fwd_b1_h2_n256_d64", "fwd", Hq=2, Hkv=2, d=64, causal=False, seed=1, B=1, N=256),
    "fwd_b4_h16_n4096_d128": Workload(
        "fwd_b4_h16_n4096_d128", "fwd", Hq=16, Hkv=16, d=128, causal=False, seed=2, B=4, N=4096),
    "fwd_causal_b2_h16_n16384_d128": Workload(
        "fwd_causal_b2_h16_n16384_d128", "fwd", Hq=16, Hkv=16, d=128, causal=True, seed=3, B=2, N=16384),
    "fwd_causal_varlen16_hq32_hkv8_d128": Workload(
        "fwd_causal_varlen16_hq32_hkv8_d128", "fwd", Hq=32, Hkv=8, d=128, causal=True, seed=4,
        B=16, varlen=True, len_lo=512, len_hi=16384),
    "bwd_causal_b2_h16_n8192_d128": Workload(
        "bwd_causal_b2_h16_n8192_d128", "bwd", Hq=16, Hkv=16, d=128, causal=True, seed=5, B=2, N=8192),
    # the packed GQA workload's shapes and Q/K/V, backward (dO drawn after V)
    "bwd_causal_varlen16_hq32_hkv8_d128": Workload(
        "bwd_causal_varlen16_hq32_hkv8_d128", "bwd", Hq=32, Hkv=8, d=128, causal=True, seed=4,
        B=16, varlen=True, len_lo=512, len_hi=16384),
    # split-KV partial results + merge: 512 queries (the last 512 positions)
    # against 131072 keys, 16 key chunks
    "split_causal_b1_hq32_hkv8_nq512_nk131072_d128": Workload(
        "split_causal_b1_hq32_hkv8_nq512_nk131072_d128", "split", Hq=32, Hkv=8, d=128, causal=True, seed=8,
        B=1, N=512, Nk=131072, n_splits=16),
    # 8-bit Q/K forward (E4M3, per-(sequence, head) descales), non-causal and causal
    "fp8_fwd_b4_h16_n4096_d128": Workload(
        "fp8_fwd_b4_h16_n4096_d128", "fp8", Hq=16, Hkv=16, d=128, causal=False, seed=9, B=4, N=4096),
    "fp8_fwd_causal_b2_h16_n16384_d128": Workload(
        "fp8_fwd_causal_b2_h16_n16384_d128", "fp8", Hq=16, Hkv=16, d=128, causal=True, seed=10, B=2, N=16384),
    # long context on one GPU
    "fwd_causal_b1_h16_n131072_d128": Workload(
        "fwd_causal_b1_h16_n131072_d128", "fwd", Hq=16, Hkv=16, d=128, causal=True, seed=6, B=1, N=131072),
    "bwd_causal_b1_h8_n65536_d128": Workload(
        "bwd_causal_b1_h8_n65536_d128", "bwd", Hq=8, Hkv=8, d=128, causal=True, seed=7, B=1, N=65536),
}


@dataclasses.dataclass
class Inputs:
    """bf16 bit patterns (uint16) for the operands, plus the packing metadata."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]   # int32 [B+1] or None
    B: int
    N: int                             # uniform length, or max length when packed
    Hq: int
    Hkv: int
    d: int
    causal: bool
    scale: float

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1]) if self.cu_seqlens is not None else self.B * self.N

    def lengths(self) -> np.ndarray:
        if self.cu_seqlens is None:
            return np.full(self.B, self.N, dtype=np.int64)
        return np.diff(self.cu_seqlens.astype(np.int64))


def _draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def draw_lengths(rng: np.random.Generator, n_seqs: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi, endpoint=True, size=n_seqs).astype(np.int64)


def make_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, causal: bool, seed: int,
                scale: Optional[float] = None, with_do: bool = False,
                lengths: Optional[np.ndarray] = None, len_range: Optional[tuple] = None,
                n_seqs: Optional[int] = None) -> Inputs:
    """Draw one seeded input set.

    Uniform batch: ``lengths`` and ``len_range`` are None, tensors are BSHD.
    Packed batch: give explicit ``lengths`` or ``len_range=(lo, hi)`` with
    ``n_seqs``; lengths are drawn first from the same generator.
    """
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    cu = None
    if len_range is not None:
        lengths = draw_lengths(rng, n_seqs, len_range[0], len_range[1])
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B = len(lengths)
        N = int(lengths.max()) if len(lengths) else 0
        T = int(cu[-1])
        qs, ks = (T, Hq, d), (T, Hkv, d)
    else:
        qs, ks = (B, N, Hq, d), (B, N, Hkv, d)
    q = _draw_bf16(rng, qs)
    k = _draw_bf16(rng, ks)
    v = _draw_bf16(rng, ks)
    do = _draw_bf16(rng, qs) if with_do else None
    return Inputs(q=q, k=k, v=v, do=do, cu_seqlens=cu, B=B, N=N, Hq=Hq, Hkv=Hkv, d=d,
                  causal=causal, scale=scale)


@dataclasses.dataclass
class SplitInputs:
    """bf16 bit patterns of a split-KV problem: Q [B, Nq, Hq, d], K/V [B, Nk, Hkv, d]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    B: int
    Nq: int
    Nk: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    scale: float
    n_splits: int


def make_split_inputs(B: int, Nq: int, Nk: int, Hq: int, Hkv: int, d: int, causal: bool, seed: int,
                      n_splits: int, scale: Optional[float] = None) -> SplitInputs:
    """Q, K, V drawn in that order, as for the other workloads."""
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    q = _draw_bf16(rng, (B, Nq, Hq, d))
    k = _draw_bf16(rng, (B, Nk, Hkv, d))
    v = _draw_bf16(rng, (B, Nk, Hkv, d))
    return SplitInputs(q=q, k=k, v=v, B=B, Nq=Nq, Nk=Nk, Hq=Hq, Hkv=Hkv, d=d, causal=causal, scale=scale,
                       n_splits=n_splits)


@dataclasses.dataclass
class Fp8Inputs:
    """Q, K as E4M3 codes (uint8) with fp32 descales per (sequence, head) or per 64-token
    block of each (sequence, head); V as bf16 bits."""
    q8: np.ndarray
    k8: np.ndarray
    v: np.ndarray
    q_descale: np.ndarray        # float32 [B, Hq], or [B, Hq, nb] per 64-token block
    k_descale: np.ndarray        # float32 [B, Hkv], or [B, Hkv, nb]
    cu_seqlens: Optional[np.ndarray]
    B: int
    N: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    scale: float


def _quantize_heads(x: np.ndarray, cu: Optional[np.ndarray], nseq: int):
    """Per-(sequence, head) descale = amax / 448 and the E4M3 codes of x / descale."""
    H = x.shape[-2]
    ds = np.ones((nseq, H), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for s in range(nseq):
        blk = x[s] if cu is None else x[int(cu[s]):int(cu[s + 1])]
        if blk.size == 0:
            continue
        amax = np.max(np.abs(blk), axis=(0, 2))                       # [H]
        ds[s] = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
        q = f32_to_e4m3_bits(blk / ds[s].astype(np.float64)[None, :, None])
        if cu is None:
            codes[s] = q
        else:
            codes[int(cu[s]):int(cu[s + 1])] = q
    return codes, ds


FP8_SCALE_BLOCK = 64     # tokens per descale block (local positions 64 j .. 64 j + 63)


def _quantize_blocks(x: np.ndarray, cu: Optional[np.ndarray], nseq: int, nb: int):
    """Per-(sequence, head, 64-token block) descale = amax / 448 and the E4M3 codes."""
    H = x.shape[-2]
    ds = np.ones((nseq, H, nb), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for s in range(nseq):
        seq = x[s] if cu is None else x[int(cu[s]):int(cu[s + 1])]
        out = np.zeros(seq.shape, dtype=np.uint8)
        for j in range(0, seq.shape[0], FP8_SCALE_BLOCK):
            blk = seq[j:j + FP8_SCALE_BLOCK]
            amax = np.max(np.abs(blk), axis=(0, 2))                   # [H]
            d = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
            ds[s, :, j // FP8_SCALE_BLOCK] = d
            out[j:j + FP8_SCALE_BLOCK] = f32_to_e4m3_bits(blk / d.astype(np.float64)[None, :, None])
        if cu is None:
            codes[s] = out
        else:
            codes[int(cu[s]):int(cu[s + 1])] = out
    return codes, ds


def make_fp8_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, causal: bool, seed: int,
                    lengths: Optional[np.ndarray] = None, scale: Optional[float] = None,
                    block_scale: bool = False, block_gain: float = 0.0) -> Fp8Inputs:
    """Q, K, V drawn as for make_inputs; Q and K quantised to E4M3 per (sequence, head), or per
    64-token block of each (sequence, head) with ``block_scale``; V to bf16. ``block_gain`` g > 0
    multiplies every 64-token block of Q and K (per head) by 2^-u, u uniform in [0, g], before
    quantisation: block descales then differ by up to 2^g while the scores only shrink (larger
    scores would make the softmax peak on single keys, where |O| reaches the largest |V| and
    bf16's output rounding alone exceeds 1e-2 above |O| = 4)."""
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, N = len(lengths), int(lengths.max()) if len(lengths) else 0
        T = int(cu[-1])
        qs, ks = (T, Hq, d), (T, Hkv, d)
    else:
        qs, ks = (B, N, Hq, d), (B, N, Hkv, d)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = _draw_bf16(rng, ks)
    if block_gain > 0:
        for x in (q, k):
            for s in range(B):
                lo, hi = (s * N, s * N + N) if cu is None else (int(cu[s]), int(cu[s + 1]))
                flat = x.reshape(-1, x.shape[-2], x.shape[-1])
                for j in range(lo, hi, FP8_SCALE_BLOCK):
                    g = np.exp2(-rng.uniform(0.0, block_gain, size=x.shape[-2])).astype(np.float32)
                    flat[j:min(j + FP8_SCALE_BLOCK, hi)] *= g[None, :, None]
    if block_scale:
        nb = (N + FP8_SCALE_BLOCK - 1) // FP8_SCALE_BLOCK
        q8, qd = _quantize_blocks(q, cu, B, nb)
        k8, kd = _quantize_blocks(k, cu, B, nb)
    else:
        q8, qd = _quantize_heads(q, cu, B)
        k8, kd = _quantize_heads(k, cu, B)
    return Fp8Inputs(q8=q8, k8=k8, v=v, q_descale=qd, k_descale=kd, cu_seqlens=cu, B=B, N=N, Hq=Hq, Hkv=Hkv,
                     d=d, causal=causal, scale=scale)


def visible_pairs(Nq: int, Nk: int, causal: bool) -> int:
    """(query, key) pairs a split-KV problem computes: query i sees keys <= i + Nk - Nq when causal."""
    if not causal:
        return Nq * Nk
    return Nq * (Nk - Nq) + Nq * (Nq + 1) // 2


def workload_inputs(name: str) -> Inputs:
    w = WORKLOADS[name]
    if w.kind == "fp8":
        return make_fp8_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, w.causal, w.seed, scale=w.scale)
    if w.kind == "split":
        return make_split_inputs(w.B, w.N, w.Nk, w.Hq, w.Hkv, w.d, w.causal, w.seed, w.n_splits, scale=w.scale)
    if w.varlen:
        return make_inputs(w.B, 0, w.Hq, w.Hkv, w.d, w.causal, w.seed, scale=w.scale,
                           with_do=(w.kind == "bwd"), len_range=(w.len_lo, w.len_hi), n_seqs=w.B)
    return make_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, w.causal, w.seed, scale=w.scale,
                       with_do=(w.kind == "bwd"))


def counted_flops(lengths, Hq: int, d: int, causal: bool, backward: bool = False) -> float:
    """Counted work: 4*Hq*d*sum(L^2), halved for causal; the backward counts 2.5x."""
    s = float(np.sum(np.asarray(lengths, dtype=np.float64) ** 2))
    f = 4.0 * Hq * d * s
    if causal:
        f *= 0.5
    if backward:
        f *= 2.5
    return f
