"""Pins for the float64 attention oracle.

Each ``pin_*`` function checks an attention implementation given as two
callables,
    fwd(q, k, v, scale, causal, cu_seqlens) -> (O, LSE)
    bwd(q, k, v, do, scale, causal, cu_seqlens) -> (dQ, dK, dV)
against something other than the implementation itself: brute force in pure
Python, closed forms, invariants of softmax attention, reductions to simpler
cases, a library routine (PyTorch's fp64 CPU attention and autograd) and
central finite differences. The same functions are run against deliberately
broken copies of the oracle to show that each plausible mistake is caught.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import bruteforce

TOL = 1e-11


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

BRUTE_CASES = [
    # (B, N, Hq, Hkv, d, causal)
    (1, 5, 1, 1, 3, False),
    (2, 7, 2, 1, 4, True),
    (1, 6, 4, 2, 8, False),
    (1, 9, 4, 2, 5, True),
    (2, 1, 2, 2, 3, True),
]
BRUTE_VARLEN = [([1, 3, 5], 4, 2, 6, True), ([4, 2, 7], 2, 1, 3, False)]


def pin_bruteforce(fwd, bwd=None):
    rng = np.random.default_rng(11)
    for (B, N, Hq, Hkv, d, causal) in BRUTE_CASES:
        q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
        scale = 0.37
        o, lse = fwd(q, k, v, scale, causal, None)
        ob, lb = bruteforce.forward(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        assert np.max(np.abs(o - np.array(ob))) < TOL, ("O vs brute force", B, N, Hq, Hkv, d, causal)
        assert np.max(np.abs(lse - np.array(lb))) < TOL, ("LSE vs brute force", B, N, Hq, Hkv, d, causal)
    for (lens, Hq, Hkv, d, causal) in BRUTE_VARLEN:
        cu = _cu(lens)
        T = int(cu[-1])
        q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
        o, lse = fwd(q, k, v, 0.5, causal, cu)
        ob, lb = bruteforce.forward(q.tolist(), k.tolist(), v.tolist(), 0.5, causal, cu.tolist())
        assert np.max(np.abs(o - np.array(ob))) < TOL, ("varlen O vs brute force", lens)
        assert np.max(np.abs(lse - np.array(lb))) < TOL, ("varlen LSE vs brute force", lens)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_closed_forms(fwd, bwd=None):
    rng = np.random.default_rng(12)
    # one key: O = V_0 and LSE = scale * q0.k0
    q, k, v = _rand(rng, 3, 1, 2, 4), _rand(rng, 3, 1, 2, 4), _rand(rng, 3, 1, 2, 4)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.3, causal, None)
        assert np.allclose(o, v, atol=TOL, rtol=0), "single key must return V_0"
        want = 0.3 * np.einsum("bnhd,bnhd->bhn", q, k)
        assert np.allclose(lse, want, atol=TOL, rtol=0), "single-key LSE"
    # identical V rows: O equals that row for every query
    B, N, H, d = 2, 6, 2, 5
    q, k = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    row = _rand(rng, B, 1, H, d)
    v = np.repeat(row, N, axis=1)
    for causal in (False, True):
        o, _ = fwd(q, k, v, 0.7, causal, None)
        assert np.allclose(o, np.repeat(row, N, axis=1), atol=TOL, rtol=0), "identical V rows"
    # all-ones V: each softmax row sums to one
    v1 = np.ones((B, N, H, d))
    o, _ = fwd(q, k, v1, 0.7, True, None)
    assert np.allclose(o, 1.0, atol=TOL, rtol=0), "softmax rows must sum to 1"
    # causal row 0: O_0 = V_0 and LSE_0 = scale * q0.k0
    v = _rand(rng, B, N, H, d)
    o, lse = fwd(q, k, v, 0.7, True, None)
    assert np.allclose(o[:, 0], v[:, 0], atol=TOL, rtol=0), "causal first row equals V_0"
    assert np.allclose(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), atol=TOL, rtol=0)
    # Q = 0: uniform weights over the visible keys
    qz = np.zeros_like(q)
    for causal in (False, True):
        o, lse = fwd(qz, k, v, 0.7, causal, None)
        for i in range(N):
            vis = i + 1 if causal else N
            assert np.allclose(o[:, i], v[:, :vis].mean(axis=1), atol=TOL, rtol=0), "Q=0 gives the mean of V"
            assert np.allclose(lse[:, :, i], math.log(vis), atol=TOL, rtol=0), "Q=0 gives LSE = ln(#keys)"
    # two keys, scalar head: O = logistic(a), LSE = ln(1 + e^a)
    for a in (-3.0, -0.25, 0.0, 1.5, 7.0):
        q2 = np.array([[[[a]], [[0.0]]]])        # [1, 2, 1, 1]; row 1 unused
        k2 = np.array([[[[0.0]], [[1.0]]]])
        v2 = np.array([[[[0.0]], [[1.0]]]])
        o, lse = fwd(q2, k2, v2, 1.0, False, None)
        assert abs(o[0, 0, 0, 0] - 1.0 / (1.0 + math.exp(-a))) < TOL, "two-key logistic"
        assert abs(lse[0, 0, 0] - math.log1p(math.exp(a))) < TOL, "two-key LSE"


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_invariants(fwd, bwd=None):
    rng = np.random.default_rng(13)
    B, N, Hq, Hkv, d = 2, 9, 4, 2, 6
    G = Hq // Hkv
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
    scale = 0.45
    for causal in (False, True):
        o, lse = fwd(q, k, v, scale, causal, None)
        for b in range(B):
            for h in range(Hq):
                g = h // G
                for i in range(N):
                    vis = i + 1 if causal else N
                    vv = v[b, :vis, g]
                    assert np.all(o[b, i, h] >= vv.min(axis=0) - TOL) and np.all(o[b, i, h] <= vv.max(axis=0) + TOL), \
                        "O must lie in the per-column range of the visible V rows"
                    smax = max(scale * float(np.dot(q[b, i, h], k[b, j, g])) for j in range(vis))
                    assert smax - TOL <= lse[b, h, i] <= smax + math.log(vis) + TOL, "max S <= LSE <= max S + ln(#keys)"
        # translating every key by u leaves O unchanged and shifts LSE by scale q.u
        u = _rand(rng, d)
        o2, lse2 = fwd(q, k + u, v, scale, causal, None)
        assert np.allclose(o2, o, atol=1e-10, rtol=0), "key translation changes O"
        shift = scale * np.einsum("bnhd,d->bhn", q, u)
        assert np.allclose(lse2, lse + shift, atol=1e-10, rtol=0), "key translation must shift LSE by scale*q.u"
        # adding c to every V entry adds c to O
        o3, lse3 = fwd(q, k, v + 2.5, scale, causal, None)
        assert np.allclose(o3, o + 2.5, atol=1e-10, rtol=0) and np.allclose(lse3, lse, atol=TOL, rtol=0)
    # joint permutation of keys and values (non-causal) leaves O and LSE unchanged
    o, lse = fwd(q, k, v, scale, False, None)
    perm = rng.permutation(N)
    o4, lse4 = fwd(q, k[:, perm], v[:, perm], scale, False, None)
    assert np.allclose(o4, o, atol=1e-12, rtol=0) and np.allclose(lse4, lse, atol=1e-12, rtol=0)
    # doubling scale equals doubling Q
    o5, lse5 = fwd(q, k, v, 2 * scale, True, None)
    o6, lse6 = fwd(2 * q, k, v, scale, True, None)
    assert np.allclose(o5, o6, atol=1e-12, rtol=0) and np.allclose(lse5, lse6, atol=1e-12, rtol=0)


def pin_logsumexp(fwd, bwd=None):
    """LSE equals a direct, correctly rounded log-sum-exp of the scaled scores."""
    rng = np.random.default_rng(14)
    B, N, H, d = 1, 8, 2, 4
    q, k, v = _rand(rng, B, N, H, d) * 3, _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    for causal in (False, True):
        _, lse = fwd(q, k, v, 0.8, causal, None)
        for h in range(H):
            for i in range(N):
                vis = i + 1 if causal else N
                sc = [0.8 * math.fsum(a * b for a, b in zip(q[0, i, h], k[0, j, h])) for j in range(vis)]
                assert abs(lse[0, h, i] - bruteforce.logsumexp_direct(sc)) < TOL


# ---------------------------------------------------------------------------
# reductions
# ---------------------------------------------------------------------------

def pin_reductions(fwd, bwd=None):
    rng = np.random.default_rng(15)
    B, N, Hq, Hkv, d = 2, 10, 6, 2, 4
    G = Hq // Hkv
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
    do = _rand(rng, B, N, Hq, d)
    for causal in (False, True):
        # grouped heads == multi-head attention with each K/V head repeated G times
        o, lse = fwd(q, k, v, 0.6, causal, None)
        kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
        o2, lse2 = fwd(q, kr, vr, 0.6, causal, None)
        assert np.allclose(o, o2, atol=1e-12, rtol=0) and np.allclose(lse, lse2, atol=1e-12, rtol=0), "GQA reduction"
        if bwd is not None:
            dq, dk, dv = bwd(q, k, v, do, 0.6, causal, None)
            dq2, dkr, dvr = bwd(q, kr, vr, do, 0.6, causal, None)
            assert np.allclose(dq, dq2, atol=1e-11, rtol=0), "GQA dQ reduction"
            assert np.allclose(dk, dkr.reshape(B, N, Hkv, G, d).sum(axis=3), atol=1e-11, rtol=0), "GQA dK group sum"
            assert np.allclose(dv, dvr.reshape(B, N, Hkv, G, d).sum(axis=3), atol=1e-11, rtol=0), "GQA dV group sum"
        # causal row i == non-causal attention of q_i over keys 0..i
        if causal:
            for i in (0, 3, N - 1):
                # attention of query i over keys 0..i, as a non-causal call
                # (the query is repeated to fill the i+1 query rows)
                qq = np.concatenate([q[:, i:i + 1]] * (i + 1), axis=1)
                oi, li = fwd(qq, k[:, :i + 1], v[:, :i + 1], 0.6, False, None)
                assert np.allclose(oi[:, 0], o[:, i], atol=1e-12, rtol=0), "causal row reduction (O)"
                assert np.allclose(li[:, :, 0], lse[:, :, i], atol=1e-12, rtol=0), "causal row reduction (LSE)"
    # packed variable length == separate uniform calls per sequence
    lens = [3, 1, 7, 5]
    cu = _cu(lens)
    T = int(cu[-1])
    qp, kp, vp = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    dop = _rand(rng, T, Hq, d)
    for causal in (False, True):
        o, lse = fwd(qp, kp, vp, 0.6, causal, cu)
        grads = bwd(qp, kp, vp, dop, 0.6, causal, cu) if bwd is not None else None
        for s, L in enumerate(lens):
            a, b = int(cu[s]), int(cu[s + 1])
            os_, ls_ = fwd(qp[None, a:b], kp[None, a:b], vp[None, a:b], 0.6, causal, None)
            assert np.allclose(o[a:b], os_[0], atol=1e-12, rtol=0), "varlen O reduction"
            assert np.allclose(lse[:, a:b], ls_[0], atol=1e-12, rtol=0), "varlen LSE reduction"
            if grads is not None:
                gs = bwd(qp[None, a:b], kp[None, a:b], vp[None, a:b], dop[None, a:b], 0.6, causal, None)
                for x, y in zip(grads, gs):
                    assert np.allclose(x[a:b], y[0], atol=1e-11, rtol=0), "varlen gradient reduction"


# ---------------------------------------------------------------------------
# library cross-check (PyTorch CPU float64)
# ---------------------------------------------------------------------------

def _torch_reference(q, k, v, do, scale, causal):
    import torch
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kr = tk.repeat_interleave(G, dim=1)
    vr = tv.repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, is_causal=causal, scale=scale)
    s = torch.matmul(tq, kr.transpose(-1, -2)) * scale
    if causal:
        N = q.shape[1]
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    tdo = torch.tensor(do, dtype=torch.float64).permute(0, 2, 1, 3)
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo)
    t = lambda x: x.detach().permute(0, 2, 1, 3).numpy()
    return t(out), lse.detach().numpy(), t(gq), t(gk), t(gv)


def pin_torch(fwd, bwd=None):
    rng = np.random.default_rng(16)
    for (B, N, Hq, Hkv, d, causal) in [(2, 33, 4, 2, 16, True), (1, 40, 2, 2, 8, False), (1, 17, 8, 1, 32, True)]:
        q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
        do = _rand(rng, B, N, Hq, d)
        o_t, lse_t, dq_t, dk_t, dv_t = _torch_reference(q, k, v, do, 0.3, causal)
        o, lse = fwd(q, k, v, 0.3, causal, None)
        assert np.allclose(o, o_t, atol=1e-12, rtol=0), "O vs torch fp64"
        assert np.allclose(lse, lse_t, atol=1e-12, rtol=0), "LSE vs torch fp64"
        if bwd is not None:
            dq, dk, dv = bwd(q, k, v, do, 0.3, causal, None)
            assert np.allclose(dq, dq_t, atol=1e-11, rtol=0), "dQ vs torch autograd"
            assert np.allclose(dk, dk_t, atol=1e-11, rtol=0), "dK vs torch autograd"
            assert np.allclose(dv, dv_t, atol=1e-11, rtol=0), "dV vs torch autograd"


# ---------------------------------------------------------------------------
# backward: finite differences and gradient invariants
# ---------------------------------------------------------------------------

def pin_finite_differences(fwd, bwd):
    """Central differences of L = sum(dO * O) match the analytic gradients."""
    rng = np.random.default_rng(17)
    cases = [((1, 5, 2, 1, 3), True, None), ((1, 4, 2, 2, 3), False, None)]
    lens = [2, 4]
    cases.append(((sum(lens), 2, 1, 3), True, _cu(lens)))
    h = 1e-6
    for shape, causal, cu in cases:
        if cu is None:
            B, N, Hq, Hkv, d = shape
            qs, ks = (B, N, Hq, d), (B, N, Hkv, d)
        else:
            T, Hq, Hkv, d = shape
            qs, ks = (T, Hq, d), (T, Hkv, d)
        q, k, v, do = _rand(rng, *qs), _rand(rng, *ks), _rand(rng, *ks), _rand(rng, *qs)
        scale = 0.55
        grads = bwd(q, k, v, do, scale, causal, cu)

        def loss(qq, kk, vv):
            return float(np.sum(do * fwd(qq, kk, vv, scale, causal, cu)[0]))

        for which, x in enumerate((q, k, v)):
            g = grads[which]
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.max(np.abs(num - g)) / max(np.max(np.abs(num)), 1e-12)
            assert err < 1e-6, ("finite differences", "QKV"[which], shape, causal, err)


def pin_gradient_invariants(fwd, bwd):
    """sum_j dK_j = 0 and sum_j dV_j = sum over the group's heads and rows of dO."""
    rng = np.random.default_rng(18)
    B, N, Hq, Hkv, d = 2, 12, 4, 2, 5
    G = Hq // Hkv
    q, k, v, do = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hq, d)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.4, causal, None)
        assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-11), "sum of dK over keys must vanish"
        want = do.reshape(B, N, Hkv, G, d).sum(axis=(1, 3))
        assert np.allclose(dv.sum(axis=1), want, atol=1e-11), "sum of dV over keys must equal sum of dO"
        # V -> V + c leaves dQ and dK unchanged (softmax is shift-free in V's direction)
        dq2, dk2, dv2 = bwd(q, k, v + 1.75, do, 0.4, causal, None)
        assert np.allclose(dq2, dq, atol=1e-11) and np.allclose(dk2, dk, atol=1e-11) and np.allclose(dv2, dv, atol=1e-11)


ALL_FWD_PINS = [pin_bruteforce, pin_closed_forms, pin_invariants, pin_logsumexp, pin_reductions, pin_torch]
ALL_BWD_PINS = [pin_finite_differences, pin_gradient_invariants, pin_reductions, pin_torch]


# ---------------------------------------------------------------------------
# row-sampled dQ (for sequences too long for whole heads)
# ---------------------------------------------------------------------------

def pin_dq_rows(dq_rows):
    """dq_rows(qh, kh, vh, doh, scale, causal, rows) equals PyTorch fp64 autograd's dQ on those rows."""
    rng = np.random.default_rng(23)
    for (N, d, causal) in [(37, 16, True), (29, 8, False)]:
        q, k, v, do = (rng.standard_normal((1, N, 1, d)) for _ in range(4))
        *_, dq_t, _, _ = _torch_reference(q, k, v, do, 0.4, causal)
        rows = np.array([0, 3, 17, N - 1])
        dq = dq_rows(q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0], 0.4, causal, rows)
        assert np.allclose(dq, dq_t[0, rows, 0], atol=1e-12, rtol=0), "row-sampled dQ vs torch autograd"


# ---------------------------------------------------------------------------
# split-KV partial results and their merge
# ---------------------------------------------------------------------------

SPLIT_CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, n_splits)
    (1, 7, 7, 2, 1, 4, True, 3),
    (2, 5, 9, 2, 2, 3, True, 4),
    (1, 3, 8, 4, 2, 5, False, 3),
    (1, 1, 9, 2, 1, 4, True, 5),
    (1, 6, 6, 1, 1, 3, True, 9),    # more chunks than keys: some are empty
]


def _torch_chunk(q, k, v, scale, causal, kb, ke):
    """LSE_p and O_p of keys kb..ke-1 by PyTorch fp64 logsumexp / softmax on masked scores."""
    import torch
    B, nq, Hq, d = q.shape
    nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tq = torch.tensor(q).permute(0, 2, 1, 3)
    tk = torch.tensor(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.tensor(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    s = torch.matmul(tq, tk.transpose(-1, -2)) * scale                     # [B, Hq, nq, nk]
    key = torch.arange(nk)[None, :]
    dead = (key < kb) | (key >= ke)
    if causal:
        dead = dead | (key > torch.arange(nq)[:, None] + (nk - nq))
    s = s.masked_fill(dead, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.nan_to_num(torch.matmul(p, tv), nan=0.0)                     # rows with no key: 0
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def pin_split(split, merge):
    """split(q, k, v, scale, causal, n) -> (O_part, LSE_part); merge(O_part, LSE_part) -> (O, LSE).

    Merged partials equal brute-force attention (pure Python) of the whole key
    range, with query i of Nq at key position i + Nk - Nq (brute force on the
    Nk-token sequence, last Nq rows); each part equals PyTorch's logsumexp /
    softmax restricted to keys p*C .. (p+1)*C - 1, C = ceil(Nk / n); rows that
    see no key of a part hold LSE = -inf, O = 0; merging one part, or a part
    with an all -inf one, gives that part back.
    """
    rng = np.random.default_rng(29)
    scale = 0.41
    for (B, nq, nk, Hq, Hkv, d, causal, n) in SPLIT_CASES:
        q, k, v = _rand(rng, B, nq, Hq, d), _rand(rng, B, nk, Hkv, d), _rand(rng, B, nk, Hkv, d)
        o_part, lse_part = split(q, k, v, scale, causal, n)
        assert o_part.shape == (n, B, nq, Hq, d) and lse_part.shape == (n, B, Hq, nq)
        o, lse = merge(o_part, lse_part)
        q_full = np.concatenate([_rand(rng, B, nk - nq, Hq, d), q], axis=1)
        ob, lb = bruteforce.forward(q_full.tolist(), k.tolist(), v.tolist(), scale, causal)
        ob = np.array(ob)[:, nk - nq:]
        lb = np.array(lb)[:, :, nk - nq:]
        assert np.max(np.abs(o - ob)) < TOL, ("merged O vs brute force", B, nq, nk, causal, n)
        assert np.max(np.abs(lse - lb)) < TOL, ("merged LSE vs brute force", B, nq, nk, causal, n)
        c = math.ceil(nk / n)
        for p in range(n):
            kb, ke = min(p * c, nk), min((p + 1) * c, nk)
            ot, lt = _torch_chunk(q, k, v, scale, causal, kb, ke)
            both_dead = np.isneginf(lt) & np.isneginf(lse_part[p])
            assert np.all(both_dead | (np.abs(lse_part[p] - lt) < TOL)), ("part LSE vs torch", p, kb, ke)
            assert np.max(np.abs(o_part[p] - ot)) < TOL, ("part O vs torch", p, kb, ke)
            dead_rows = np.isneginf(lse_part[p])                            # [B, Hq, nq]
            assert np.all(o_part[p].transpose(0, 2, 1, 3)[dead_rows] == 0.0), "dead rows must hold O = 0"
        o1, l1 = merge(o_part[:1], lse_part[:1])
        assert np.array_equal(l1, lse_part[0]) and np.array_equal(o1, o_part[0]), "merge of one part"
    # a part that is -inf everywhere leaves the other untouched
    o_a = _rand(rng, 1, 3, 2, 4)
    l_a = _rand(rng, 1, 2, 3)
    o_m, l_m = merge(np.stack([o_a, np.zeros_like(o_a)]), np.stack([l_a, np.full_like(l_a, -np.inf)]))
    assert np.array_equal(l_m, l_a) and np.allclose(o_m, o_a, rtol=0, atol=1e-15), "merge with an empty part"


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) Q/K forward
# ---------------------------------------------------------------------------

# Values the OCP 8-bit floating point specification states for E4M3:
# largest normal 448 (S.1111.110), smallest normal 2^-6 (S.0001.000),
# largest subnormal 0.875 * 2^-6, smallest subnormal 2^-9, 1.0 (bias 7),
# NaN for S.1111.111, and no infinities.
E4M3_FIXED = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x07: 0.875 * 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0,
              0x00: 0.0, 0xFE: -448.0, 0xBE: -1.75, 0xC0: -2.0, 0x3C: 1.5, 0x3F: 1.875, 0x40: 2.0}


def _e4m3_py(code: int) -> float:
    """Brute-force decode: the E4M3 value set enumerated binade by binade with math.ldexp."""
    mag = code & 0x7F
    table = [math.ldexp(m, -9) for m in range(8)]                        # subnormals and zero
    for e in range(1, 16):
        table += [math.ldexp(8 + m, e - 10) for m in range(8)]           # (1 + m/8) 2^(e-7)
    v = table[mag]
    return -v if code & 0x80 else v


def pin_fp8(fwd8, decode):
    """decode(bits) -> float64; fwd8(q8, k8, v, qd, kd, scale, causal, cu) -> (O, LSE).

    The decoder matches the specification's stated values, is odd-symmetric,
    strictly increasing over the finite positive codes with spacing 2^(e-10) in
    binade e, and gives NaN exactly for S.1111.111. The forward equals brute
    force (pure Python) on inputs dequantised code by code with their own
    (sequence, head) scale, uniform and packed.
    """
    codes = np.arange(256, dtype=np.uint8)
    vals = decode(codes)
    for c, want in E4M3_FIXED.items():
        assert vals[c] == want, ("E4M3 value", hex(c), vals[c], want)
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and np.sum(np.isnan(vals)) == 2, "E4M3 NaN codes"
    pos = vals[1:0x7F]
    assert np.all(np.diff(pos) > 0), "E4M3 positive codes must increase"
    assert np.all(vals[0x80:0xFF] == -vals[0:0x7F]), "E4M3 sign symmetry"
    for e in range(1, 15):
        seg = vals[8 * e: 8 * e + 8]
        assert np.all(np.diff(seg) == 2.0 ** (e - 10)), ("E4M3 spacing", e)
    assert all(vals[c] == _e4m3_py(c) for c in range(256) if (c & 0x7F) != 0x7F), "E4M3 vs enumeration"

    rng = np.random.default_rng(31)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for (B, N, Hq, Hkv, d, causal, lens) in [(2, 6, 4, 2, 5, True, None), (1, 7, 2, 1, 4, False, None),
                                             (0, 0, 4, 2, 3, True, [3, 5, 1])]:
        if lens is None:
            qs, ks, nseq = (B, N, Hq, d), (B, N, Hkv, d), B
            cu = None
        else:
            T = sum(lens)
            qs, ks, nseq = (T, Hq, d), (T, Hkv, d), len(lens)
            cu = _cu(lens)
        q8 = rng.choice(finite, size=qs)
        k8 = rng.choice(finite, size=ks)
        v = _rand(rng, *ks)
        qd = rng.uniform(0.002, 0.02, size=(nseq, Hq))
        kd = rng.uniform(0.002, 0.02, size=(nseq, Hkv))
        scale = 0.3
        o, lse = fwd8(q8, k8, v, qd, kd, scale, causal, cu)
        # dequantise code by code, each row with its own sequence's scales
        qf = np.zeros(qs)
        kf = np.zeros(ks)
        for idx in np.ndindex(*qs):
            s = idx[0] if cu is None else int(np.searchsorted(cu, idx[0], side="right") - 1)
            qf[idx] = _e4m3_py(int(q8[idx])) * qd[s, idx[-2]]
        for idx in np.ndindex(*ks):
            s = idx[0] if cu is None else int(np.searchsorted(cu, idx[0], side="right") - 1)
            kf[idx] = _e4m3_py(int(k8[idx])) * kd[s, idx[-2]]
        if cu is None:
            ob, lb = bruteforce.forward(qf.tolist(), kf.tolist(), v.tolist(), scale, causal)
        else:
            ob, lb = bruteforce.forward(qf.tolist(), kf.tolist(), v.tolist(), scale, causal, cu.tolist())
        assert np.max(np.abs(o - np.array(ob))) < TOL, ("FP8 O vs brute force", B, N, causal, lens)
        assert np.max(np.abs(lse - np.array(lb))) < TOL, ("FP8 LSE vs brute force", B, N, causal, lens)


def pin_fp8_blocks(fwd8):
    """Block-scaled 8-bit inputs: one descale per 64-token block of each (sequence, head),
    block t // 64 for the token at local position t. The forward equals brute force (pure
    Python) on inputs dequantised code by code, each element with the scale its sequence,
    head and local position select, uniform and packed (sequences of 1 to 3 blocks, one
    ending mid-block); and block descales that are all equal give exactly the result of
    the per-(sequence, head) descales."""
    rng = np.random.default_rng(37)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for (B, N, Hq, Hkv, d, causal, lens) in [(1, 150, 2, 1, 3, True, None), (2, 70, 2, 2, 2, False, None),
                                             (0, 0, 2, 2, 2, False, [70, 130, 5])]:
        if lens is None:
            qs, ks, nseq, nmax = (B, N, Hq, d), (B, N, Hkv, d), B, N
            cu = None
        else:
            T = sum(lens)
            qs, ks, nseq, nmax = (T, Hq, d), (T, Hkv, d), len(lens), max(lens)
            cu = _cu(lens)
        nb = (nmax + 63) // 64
        q8 = rng.choice(finite, size=qs)
        k8 = rng.choice(finite, size=ks)
        v = _rand(rng, *ks)
        qd = rng.uniform(0.002, 0.02, size=(nseq, Hq, nb))
        kd = rng.uniform(0.002, 0.02, size=(nseq, Hkv, nb))
        scale = 0.3
        o, lse = fwd8(q8, k8, v, qd, kd, scale, causal, cu)

        def deq(codes, desc, shape):
            out = np.zeros(shape)
            for idx in np.ndindex(*shape):
                if cu is None:
                    s, pos = idx[0], idx[1]
                else:
                    s = int(np.searchsorted(cu, idx[0], side="right") - 1)
                    pos = idx[0] - int(cu[s])
                out[idx] = _e4m3_py(int(codes[idx])) * desc[s, idx[-2], pos // 64]
            return out
        qf, kf = deq(q8, qd, qs), deq(k8, kd, ks)
        if cu is None:
            ob, lb = bruteforce.forward(qf.tolist(), kf.tolist(), v.tolist(), scale, causal)
        else:
            ob, lb = bruteforce.forward(qf.tolist(), kf.tolist(), v.tolist(), scale, causal, cu.tolist())
        assert np.max(np.abs(o - np.array(ob))) < TOL, ("FP8 block O vs brute force", B, N, causal, lens)
        assert np.max(np.abs(lse - np.array(lb))) < TOL, ("FP8 block LSE vs brute force", B, N, causal, lens)
        # equal blocks reduce to per-(sequence, head) descales
        o1, l1 = fwd8(q8, k8, v, qd[:, :, :1].repeat(nb, axis=2), kd[:, :, :1].repeat(nb, axis=2), scale, causal, cu)
        o2, l2 = fwd8(q8, k8, v, qd[:, :, 0], kd[:, :, 0], scale, causal, cu)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "equal block descales != per-head descales"


def pin_rowdot(rowdot):
    """D_i = dO_i . O_i equals sum_j P_ij dP_ij with dP_ij = dO_i . V_j (O_i = sum_j P_ij V_j):
    P and O from the pure-Python brute force, the double sum in math.fsum, for uniform and
    packed layouts ([B, Hq, N] and [Hq, T]), causal, with grouped K/V heads."""
    from oracle import bruteforce as bf
    rng = np.random.default_rng(4)
    for cu in (None, np.array([0, 3, 3, 7], dtype=np.int32)):
        shp_q, shp_k = ((2, 5, 4, 3), (2, 5, 2, 3)) if cu is None else ((7, 4, 3), (7, 2, 3))
        q, k, v = rng.standard_normal(shp_q), rng.standard_normal(shp_k), rng.standard_normal(shp_k)
        do = rng.standard_normal(shp_q)
        o, _ = bf.forward(q.tolist(), k.tolist(), v.tolist(), 0.7, True, None if cu is None else cu.tolist())
        o = np.array(o)
        d = rowdot(do, o)
        seqs = [(b, b, 5) for b in range(2)] if cu is None else [(s, int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(3)]
        for s, start, L in seqs:
            for h in range(4):
                g = h // 2
                for i in range(L):
                    row = (lambda x, j: x[s, j, h]) if cu is None else (lambda x, j: x[start + j, h])
                    krow = (lambda x, j: x[s, j, g]) if cu is None else (lambda x, j: x[start + j, g])
                    sc = [0.7 * math.fsum(a * b for a, b in zip(row(q, i), krow(k, j))) for j in range(i + 1)]
                    m = max(sc)
                    e = [math.exp(x - m) for x in sc]
                    z = math.fsum(e)
                    dp = [math.fsum(a * b for a, b in zip(row(do, i), krow(v, j))) for j in range(i + 1)]
                    want = math.fsum(e[j] / z * dp[j] for j in range(i + 1))
                    got = d[s, h, i] if cu is None else d[h, start + i]
                    assert abs(got - want) <= 1e-12 * (1 + abs(want)), (cu is None, s, h, i, got, want)
