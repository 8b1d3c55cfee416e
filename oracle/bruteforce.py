"""Pure-Python brute-force attention for tiny inputs (test infrastructure).

An independent second route to the same definition as ``oracle.attention``:
nested Python loops over plain floats, ``math.exp`` and correctly rounded
``math.fsum`` sums, no NumPy arithmetic. Used only by the tests to pin the
NumPy oracle on tiny shapes. The definition it follows is the exact softmax
attention of FlashAttention (reference 2 on the podcast.app episode page,
"FlashAttention: Fast and Memory-Efficient Exact Attention with
IO-Awareness"), with causal masking and packed variable-length batches as
named in the daily.dev "Summary".

Inputs are nested lists (or arrays converted with ``.tolist()``) in the same
layouts as ``oracle.attention``.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence


def _sequences(n_batch: int, seq_len: int, cu_seqlens: Optional[Sequence[int]]):
    if cu_seqlens is None:
        return [(b, None, seq_len) for b in range(n_batch)]
    return [(s, int(cu_seqlens[s]), int(cu_seqlens[s + 1]) - int(cu_seqlens[s]))
            for s in range(len(cu_seqlens) - 1)]


def _row(x, s, start, i, h):
    """The d-vector of token i (local) of sequence s, head h."""
    return x[start + i][h] if start is not None else x[s][i][h]


def forward(q, k, v, scale: float, causal: bool, cu_seqlens: Optional[Sequence[int]] = None):
    """Return (O, LSE) as nested lists shaped like the NumPy oracle's outputs."""
    packed = cu_seqlens is not None
    if packed:
        T = len(q)
        Hq = len(q[0]) if T else 0
        Hkv = len(k[0]) if T else 1
        d = len(q[0][0]) if T else 0
        o = [[[math.nan] * d for _ in range(Hq)] for _ in range(T)]
        lse = [[math.nan] * T for _ in range(Hq)]
        seqs = _sequences(0, 0, cu_seqlens)
    else:
        B, N = len(q), len(q[0])
        Hq, Hkv, d = len(q[0][0]), len(k[0][0]), len(q[0][0][0])
        o = [[[[math.nan] * d for _ in range(Hq)] for _ in range(N)] for _ in range(B)]
        lse = [[[math.nan] * N for _ in range(Hq)] for _ in range(B)]
        seqs = _sequences(B, N, None)
    G = Hq // Hkv
    for s, start, L in seqs:
        for h in range(Hq):
            g = h // G
            for i in range(L):
                qi = _row(q, s, start, i, h)
                scores: List[float] = []
                for j in range(L):
                    if causal and j > i:
                        continue
                    kj = _row(k, s, start, j, g)
                    scores.append(scale * math.fsum(a * b for a, b in zip(qi, kj)))
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                total = math.fsum(w)
                out = []
                for c in range(d):
                    out.append(math.fsum(w[j] * _row(v, s, start, j, g)[c] for j in range(len(w))) / total)
                lse_i = m + math.log(total)
                if packed:
                    o[start + i][h] = out
                    lse[h][start + i] = lse_i
                else:
                    o[s][i][h] = out
                    lse[s][h][i] = lse_i
    return o, lse


def logsumexp_direct(values: Sequence[float]) -> float:
    """ln(sum(exp(x))) summed with fsum, shifted by the max for range safety."""
    m = max(values)
    return m + math.log(math.fsum(math.exp(x - m) for x in values))
