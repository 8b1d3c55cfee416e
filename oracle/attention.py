"""CPU reference for exact softmax attention, in float64 (test infrastructure).

This module is the oracle that the HIP kernels are checked against. It is
test infrastructure only: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the library never does.

What it computes is the plain definition of exact attention, the result that
FlashAttention's tiling with an online softmax reaches without ever writing
the N x N score matrix to memory ("FlashAttention-4 Conquers Asymmetric GPU
Hardware Scaling", podcast.app episode page, second paragraph of the
description; reference 2 there, "FlashAttention: Fast and Memory-Efficient
Exact Attention with IO-Awareness"). Because the tiled method is exact, the
oracle materialises S and P in full instead of tiling, and shares nothing
with the GPU path.

For one sequence of length L, one query head h and its key/value head
g = h // (Hq // Hkv):
  S[i, j] = scale * sum_k Q[i, h, k] K[j, g, k]; with causal masking
            S[i, j] = -inf for j > i (positions local to the sequence)
  m_i     = max_j S[i, j]
  l_i     = sum_j exp(S[i, j] - m_i)
  P[i, j] = exp(S[i, j] - m_i) / l_i
  O[i]    = sum_j P[i, j] V[j, g]
  LSE_i   = m_i + ln(l_i)          (natural log of sum_j exp(S[i, j]))
Backward, for an upstream gradient dO (the backward pass named in the
abstract on the zhuanzhiai.com page):
  dV[j, g] = sum over heads h of group g, sum_i P[i, j] dO[i, h]
  dP[i, j] = dO[i, h] . V[j, g]
  D_i      = dO[i, h] . O[i, h]
  dS[i, j] = P[i, j] (dP[i, j] - D_i)
  dQ[i, h] = scale * sum_j dS[i, j] K[j, g]
  dK[j, g] = scale * sum over heads h of group g, sum_i dS[i, j] Q[i, h]

Layouts (contiguous "BSHD"): uniform batches Q/O/dO [B, N, Hq, d] and K/V
[B, N, Hkv, d], LSE [B, Hq, N]; packed variable-length batches (the
cu_seqlens form; the daily.dev summary names variable sequence lengths)
Q [T, Hq, d], K/V [T, Hkv, d], LSE [Hq, T], sequence s occupying rows
cu_seqlens[s] .. cu_seqlens[s+1]-1.

Inputs are float64 arrays (the exact values of the bf16 operands).
"""
from __future__ import annotations

from typing import Callable, Iterator, Optional, Tuple

import numpy as np

RowSelect = Optional[Callable[[int, int], np.ndarray]]


def _segments(q: np.ndarray, cu_seqlens: Optional[np.ndarray]) -> Iterator[Tuple[int, slice, int]]:
    """Yield (sequence index, token slice, length) for each sequence.

    Uniform batches ([B, N, H, d]) yield batch indices with slice(None);
    packed batches ([T, H, d]) yield row ranges of the packed tensor.
    """
    if cu_seqlens is None:
        for b in range(q.shape[0]):
            yield b, slice(None), q.shape[1]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for s in range(len(cu) - 1):
            yield s, slice(int(cu[s]), int(cu[s + 1])), int(cu[s + 1] - cu[s])


def _seq(x: np.ndarray, s: int, sl: slice, packed: bool) -> np.ndarray:
    """The [L, H, d] block of sequence s."""
    return x[sl] if packed else x[s]


def head_scores(qh: np.ndarray, kh: np.ndarray, scale: float, causal: bool,
                rows: Optional[np.ndarray] = None) -> np.ndarray:
    """S = scale * Q K^T for one head, with -inf above the diagonal when causal.

    qh [L, d], kh [L, d]; ``rows`` (local query indices) restricts the rows.
    """
    if rows is None:
        rows = np.arange(qh.shape[0])
    s = scale * (qh[rows] @ kh.T)
    if causal:
        j = np.arange(kh.shape[0])
        s[j[None, :] > rows[:, None]] = -np.inf
    return s


def head_forward(qh, kh, vh, scale, causal, rows=None):
    """Softmax attention for one (sequence, head): returns (O [R, d], LSE [R], P [R, L])."""
    s = head_scores(qh, kh, scale, causal, rows)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ vh
    lse = m + np.log(l)
    return o, lse, p


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      causal: bool, cu_seqlens: Optional[np.ndarray] = None,
                      rows: RowSelect = None):
    """Exact attention forward. Returns (O, LSE) in float64.

    ``rows(s, L)`` may return the local query rows of sequence s to compute;
    rows not computed are NaN in the outputs (used for sampled checks of very
    long sequences, where every computed row is still exact).
    """
    packed = cu_seqlens is not None
    Hq, Hkv = q.shape[-2], k.shape[-2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.full(q.shape, np.nan, dtype=np.float64)
    if packed:
        lse = np.full((Hq, q.shape[0]), np.nan, dtype=np.float64)
    else:
        lse = np.full((q.shape[0], Hq, q.shape[1]), np.nan, dtype=np.float64)
    for s, sl, L in _segments(q, cu_seqlens):
        if L == 0:
            continue
        qs, ks, vs = _seq(q, s, sl, packed), _seq(k, s, sl, packed), _seq(v, s, sl, packed)
        r = np.arange(L) if rows is None else np.asarray(rows(s, L), dtype=np.int64)
        for h in range(Hq):
            g = h // G
            oh, lh, _ = head_forward(qs[:, h, :], ks[:, g, :], vs[:, g, :], scale, causal, r)
            if packed:
                o[sl.start + r, h, :] = oh
                lse[h, sl.start + r] = lh
            else:
                o[s, r, h, :] = oh
                lse[s, h, r] = lh
    return o, lse


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       scale: float, causal: bool, cu_seqlens: Optional[np.ndarray] = None):
    """Gradients of the exact attention output. Returns (dQ, dK, dV) in float64.

    O, P and D are the oracle's own float64 values, recomputed from Q, K, V.
    """
    packed = cu_seqlens is not None
    Hq, Hkv = q.shape[-2], k.shape[-2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for s, sl, L in _segments(q, cu_seqlens):
        if L == 0:
            continue
        qs, ks, vs = _seq(q, s, sl, packed), _seq(k, s, sl, packed), _seq(v, s, sl, packed)
        dos = _seq(do, s, sl, packed)
        dqs, dks, dvs = _seq(dq, s, sl, packed), _seq(dk, s, sl, packed), _seq(dv, s, sl, packed)
        for h in range(Hq):
            g = h // G
            gq, gk, gv = head_backward(qs[:, h, :], ks[:, g, :], vs[:, g, :], dos[:, h, :], scale, causal)
            dqs[:, h, :] += gq
            dks[:, g, :] += gk
            dvs[:, g, :] += gv
    return dq, dk, dv


def head_backward(qh, kh, vh, doh, scale, causal):
    """Gradients for one (sequence, query head): returns (dQ [L, d], dK [L, d], dV [L, d])."""
    oh, _, p = head_forward(qh, kh, vh, scale, causal)
    dv = p.T @ doh
    dp = doh @ vh.T
    d_row = np.sum(doh * oh, axis=1)
    ds = p * (dp - d_row[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def head_backward_dq_rows(qh, kh, vh, doh, scale, causal, rows):
    """dQ of the selected rows of one (sequence, query head): [R, d].

    Row i of dQ needs only row i of P, O and dO (the dS and dQ lines of the
    definition above, for one i): P_i and O_i from the row-restricted forward,
    dP_i = dO_i V^T, D_i = dO_i . O_i, dS_i = P_i (dP_i - D_i), dQ_i = scale dS_i K.
    Used for sampled checks of sequences too long for whole heads.
    """
    rows = np.asarray(rows, dtype=np.int64)
    o_r, _, p_r = head_forward(qh, kh, vh, scale, causal, rows)
    do_r = doh[rows]
    dp_r = do_r @ vh.T
    dd_r = np.sum(do_r * o_r, axis=1)
    ds_r = p_r * (dp_r - dd_r[:, None])
    return scale * (ds_r @ kh)


def backward_rowdot(do: np.ndarray, o: np.ndarray) -> np.ndarray:
    """D_i = sum_k dO[i, h, k] O[i, h, k], shaped like the LSE ([B, Hq, N] or [Hq, T])."""
    d = np.sum(do * o, axis=-1)
    if d.ndim == 3:
        return np.transpose(d, (0, 2, 1)).copy()
    return d.T.copy()


# ---------------------------------------------------------------------------
# Split-KV partial results and their merge.
#
# Attention over all keys equals the merge of attention over disjoint key
# chunks: with LSE_p the log-sum-exp of the scores of chunk p and O_p that
# chunk's softmax-weighted sum of V, LSE = ln sum_p exp(LSE_p) and
# O = sum_p exp(LSE_p - LSE) O_p. This is the combination step of the online
# softmax that tiling relies on (podcast.app episode page, description,
# second paragraph), applied across chunks instead of tiles; the same step
# joins the partial results of blockwise ring attention (that page's source
# list, "Ring Attention with Blockwise Transformers for Near-Infinite
# Context"). The pages give no layout or chunking for it; the readings here:
#   * queries and keys may differ in number (Nq <= Nk when causal); query i
#     sits at key position i + Nk - Nq, so the last query sees every key;
#   * chunk p holds keys p*C .. min((p+1)*C, Nk) - 1 with C = ceil(Nk / n);
#   * a row that sees no key of a chunk has LSE_p = -inf and O_p = 0.
# ---------------------------------------------------------------------------

def split_chunk(nk: int, n_splits: int, p: int) -> Tuple[int, int]:
    """Key range [begin, end) of chunk p (empty when begin >= end)."""
    c = -(-nk // n_splits)
    return min(p * c, nk), min((p + 1) * c, nk)


def head_forward_keys(qh, kh, vh, scale, causal, q_off, kb, ke):
    """Attention of every query of one head over keys kb .. ke-1 only.

    qh [Nq, d], kh/vh [Nk, d]; query i is at key position i + q_off. Returns
    (O [Nq, d], LSE [Nq]) with O = 0, LSE = -inf for rows seeing no key.
    """
    nq = qh.shape[0]
    o = np.zeros((nq, qh.shape[1]))
    lse = np.full(nq, -np.inf)
    if ke <= kb:
        return o, lse
    s = scale * (qh @ kh[kb:ke].T)
    if causal:
        j = np.arange(kb, ke)
        s[j[None, :] > (np.arange(nq) + q_off)[:, None]] = -np.inf
    live = np.isfinite(s).any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1)
        e = np.exp(sl - m[:, None])
        l = e.sum(axis=1)
        o[live] = (e / l[:, None]) @ vh[kb:ke]
        lse[live] = m + np.log(l)
    return o, lse


def attention_forward_split(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                            n_splits: int):
    """Partial attention over each of n_splits key chunks (uniform batches).

    Q [B, Nq, Hq, d], K/V [B, Nk, Hkv, d]. Returns O_part [n, B, Nq, Hq, d]
    and LSE_part [n, B, Hq, Nq] in float64 (readings above).
    """
    B, nq, Hq, d = q.shape
    nk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and nq > nk:
        raise ValueError("causal needs Nq <= Nk")
    G = Hq // Hkv
    o_part = np.zeros((n_splits, B, nq, Hq, d))
    lse_part = np.full((n_splits, B, Hq, nq), -np.inf)
    for p in range(n_splits):
        kb, ke = split_chunk(nk, n_splits, p)
        for b in range(B):
            for h in range(Hq):
                g = h // G
                oh, lh = head_forward_keys(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], scale, causal,
                                           nk - nq, kb, ke)
                o_part[p, b, :, h, :] = oh
                lse_part[p, b, h, :] = lh
    return o_part, lse_part


def merge_partials(o_part: np.ndarray, lse_part: np.ndarray):
    """Merge partial results: LSE = ln sum_p exp(LSE_p), O = sum_p exp(LSE_p - LSE) O_p.

    o_part [n, B, N, H, d], lse_part [n, B, H, N]; rows whose every LSE_p is
    -inf get LSE = -inf and O = 0. Returns (O [B, N, H, d], LSE [B, H, N]).
    """
    m = lse_part.max(axis=0)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    w = np.exp(lse_part - m_safe[None])                     # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, tot)))
    coef = np.where(dead[None], 0.0, w / np.where(dead, 1.0, tot)[None])   # [n, B, H, N]
    o = np.einsum("pbhn,pbnhd->bnhd", coef, o_part)
    return o, lse


# ---------------------------------------------------------------------------
# FP8 forward: Q and K in 8-bit floating point with per-(sequence, head)
# scales, V in bf16.
#
# The pages name low-precision attention in FlashAttention's lineage
# (podcast.app episode page, source list: "FlashAttention-3: Fast and Accurate
# Attention with Asynchrony and Low Precision", and SageAttention2, which
# quantises Q and K more coarsely than the P V product). They fix no format.
# The reading here: Q and K are OCP E4M3 values (1 sign, 4 exponent bits with
# bias 7, 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN;
# no infinities; largest finite 448), dequantised as x = e4m3 * descale with
# one fp32 descale per (sequence, head); V stays bf16. What is computed is the
# exact attention of those dequantised values.
# ---------------------------------------------------------------------------

def e4m3_to_float(bits: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 bit patterns (uint8) to float64."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * val
    return np.where((b & 0x7F) == 0x7F, np.nan, out)


# Tokens per descale block of the block-scaled 8-bit inputs: block j of a
# sequence holds its tokens 64 j .. 64 j + 63 (positions local to the sequence).
FP8_SCALE_BLOCK = 64


def _token_descales(desc: np.ndarray, n_tokens: int) -> np.ndarray:
    """Descale of every token of one sequence, [n_tokens, H], from one sequence's
    descales: [H] (one per head) or [H, nb] (one per head and 64-token block)."""
    desc = np.asarray(desc, dtype=np.float64)
    if desc.ndim == 1:
        return np.broadcast_to(desc[None, :], (n_tokens, desc.shape[0]))
    block = np.arange(n_tokens) // FP8_SCALE_BLOCK
    return desc[:, block].T


def attention_forward_fp8(q8: np.ndarray, k8: np.ndarray, v: np.ndarray, q_descale: np.ndarray,
                          k_descale: np.ndarray, scale: float, causal: bool,
                          cu_seqlens: Optional[np.ndarray] = None, rows: RowSelect = None):
    """Exact attention of the dequantised FP8 inputs. Returns (O, LSE) in float64.

    q8, k8: uint8 E4M3 in the Q / K layouts; v: float64 values in the V layout.
    Descales, B = number of sequences when packed: per (sequence, head),
    q_descale [B, Hq] and k_descale [B, Hkv]; or per 64-token block of each
    (sequence, head), q_descale [B, Hq, nb] and k_descale [B, Hkv, nb], where
    token t of a sequence (local position) uses block t // 64. An element's
    value is its code times its descale.
    """
    packed = cu_seqlens is not None
    q = e4m3_to_float(q8)
    k = e4m3_to_float(k8)
    qd = np.asarray(q_descale, dtype=np.float64)
    kd = np.asarray(k_descale, dtype=np.float64)
    if packed:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for s in range(len(cu) - 1):
            L = int(cu[s + 1] - cu[s])
            q[cu[s]:cu[s + 1]] *= _token_descales(qd[s], L)[:, :, None]
            k[cu[s]:cu[s + 1]] *= _token_descales(kd[s], L)[:, :, None]
    else:
        for b in range(q.shape[0]):
            q[b] *= _token_descales(qd[b], q.shape[1])[:, :, None]
            k[b] *= _token_descales(kd[b], k.shape[1])[:, :, None]
    return attention_forward(q, k, v, scale, causal, cu_seqlens, rows)
