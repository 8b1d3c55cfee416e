"""Split-KV partial results and the log-sum-exp merge on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_48_amd import capi, inputs as I, ops
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# (B, Nq, Nk, Hq, Hkv, d, causal, n_splits)
SPLIT_CASES = [
    (1, 300, 300, 2, 1, 64, True, 3),       # Nq = Nk; 100-key chunks (not a tile multiple)
    (2, 129, 700, 4, 2, 128, True, 4),      # the last 129 positions against 700 keys
    (1, 1, 1000, 8, 2, 128, True, 7),       # one query (decoding)
    (1, 257, 513, 2, 2, 128, False, 5),     # ragged, no mask
    (1, 64, 64, 2, 1, 128, True, 9),        # 8-key chunks; early rows see nothing of later chunks
    (1, 33, 40, 2, 2, 64, False, 16),       # 3-key chunks: the last two chunks are empty
    (1, 520, 4100, 4, 4, 128, True, 1),     # one chunk: plain attention in fp32 partial form
    (1, 33, 40, 2, 2, 128, False, 16),      # d = 128 with empty trailing chunks
    (1, 300, 100, 2, 1, 128, False, 3),     # more queries than keys (no mask)
    (2, 600, 1300, 4, 2, 128, True, 5),     # three query tiles, causal offset 700 across 260-key chunks
    (1, 64, 20000, 2, 1, 128, True, 1),     # one chunk of 313 key tiles (past a 256-tile copy window)
]


def _ids(c):
    return "B{}_Nq{}_Nk{}_Hq{}_Hkv{}_d{}_{}_n{}".format(*c[:6], "causal" if c[6] else "full", c[7])


def _check_parts(o_part, lse_part, o_ref, lse_ref, label):
    """fp32 partials: O max-abs and LSE max-abs as for the forward; -inf exactly where the oracle has it."""
    o = H.host_f64(o_part)
    lse = H.host_f64(lse_part)
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), dead), f"{label}: -inf LSE pattern differs"
    assert np.all(np.isfinite(lse[~dead])) and np.all(np.isfinite(o)), f"{label}: non-finite partials"
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~dead] - lse_ref[~dead]))) if (~dead).any() else 0.0
    assert eo <= H.O_MAX_ABS, f"{label}: O_p max-abs error {eo:.3e}"
    assert el <= H.LSE_MAX_ABS, f"{label}: LSE_p max-abs error {el:.3e}"


@pytest.mark.parametrize("case", SPLIT_CASES, ids=_ids)
def test_split_and_merge(case):
    B, Nq, Nk, Hq, Hkv, d, causal, n = case
    x = I.make_split_inputs(B, Nq, Nk, Hq, Hkv, d, causal, seed=300 + Nq + n, n_splits=n)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    o_part, lse_part = ops.forward_split(q, k, v, causal, n, x.scale)
    o, lse = ops.merge(o_part, lse_part)
    torch.cuda.synchronize()
    op_ref, lp_ref = oracle.attention_forward_split(H.f64(x.q), H.f64(x.k), H.f64(x.v), x.scale, causal, n)
    _check_parts(o_part, lse_part, op_ref, lp_ref, _ids(case))
    o_ref, lse_ref = oracle.merge_partials(op_ref, lp_ref)
    H.check_forward(o, lse, o_ref, lse_ref, _ids(case) + " merged")


def test_split_of_self_attention_matches_forward():
    """Nq = Nk: the merged split result and fa_fwd agree to the forward's tolerance (both against the oracle)."""
    x = I.make_inputs(2, 777, 4, 2, 128, True, seed=61)
    q, k, v, _, o_f, lse_f = H.gpu_forward(x)
    o, lse = ops.merge(*ops.forward_split(q, k, v, True, 6, x.scale))
    torch.cuda.synchronize()
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, "split 6 + merge")
    H.check_forward(o_f, lse_f, o_ref, lse_ref, "fa_fwd")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_parts", [1, 2, 5])
def test_merge_matches_oracle(d, n_parts):
    """Partials from a seeded host draw (not from the GPU path), some rows -inf in some or all parts."""
    rng = np.random.default_rng(70 + d + n_parts)
    B, N, Hh = 2, 77, 3
    o_part = rng.standard_normal((n_parts, B, N, Hh, d)).astype(np.float32)
    lse_part = (rng.standard_normal((n_parts, B, Hh, N)) * 4).astype(np.float32)
    lse_part[:, 0, 0, :5] = -np.inf                         # rows dead in every part
    lse_part[0, 1, 2, 10:20] = -np.inf                      # dead in one part
    for p in range(n_parts):                                # dead parts hold O_p = 0
        o_part[p][np.isneginf(lse_part[p]).transpose(0, 2, 1)] = 0.0
    o_ref, lse_ref = oracle.merge_partials(o_part.astype(np.float64), lse_part.astype(np.float64))
    o, lse = ops.merge(torch.from_numpy(o_part).cuda(), torch.from_numpy(lse_part).cuda())
    torch.cuda.synchronize()
    og, lg = H.host_f64(o), H.host_f64(lse)
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), dead)
    assert np.max(np.abs(lg[~dead] - lse_ref[~dead])) < 1e-5
    # bf16 output: within half an ulp of bf16 (2^-9 relative) plus fp32 rounding
    err = np.abs(og - o_ref)
    assert np.all(err <= np.abs(o_ref) * 2.0 ** -8 + 1e-6), float(np.max(err / (np.abs(o_ref) + 1e-6)))
    assert np.all(og[dead.transpose(0, 2, 1)] == 0.0)


def test_split_workload_sampled():
    """split_causal_b1_hq32_hkv8_nq512_nk131072_d128 at full size with the bench's launch (16 chunks):
    sampled rows of a few heads against the oracle, one row at a time, for each part and merged."""
    w = I.WORKLOADS["split_causal_b1_hq32_hkv8_nq512_nk131072_d128"]
    x = I.workload_inputs(w.name)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    o_part, lse_part = ops.forward_split(q, k, v, x.causal, x.n_splits, x.scale)
    o, lse = ops.merge(o_part, lse_part)
    torch.cuda.synchronize()
    op, lp, og, lg = (H.host_f64(t) for t in (o_part, lse_part, o, lse))
    kf, vf = H.f64(x.k[0]), H.f64(x.v[0])
    G = x.Hq // x.Hkv
    for h in (0, 13, x.Hq - 1):
        g = h // G
        for r in (0, 1, 255, 256, 400, x.Nq - 1):
            qrow = H.f64(x.q[0, r:r + 1, h])
            q_off = r + x.Nk - x.Nq
            for p in (0, 7, x.n_splits - 1):
                kb, ke = oracle.split_chunk(x.Nk, x.n_splits, p)
                o_r, l_r = oracle.head_forward_keys(qrow, kf[:, g], vf[:, g], x.scale, True, q_off, kb, ke)
                assert abs(lp[p, 0, h, r] - l_r[0]) <= H.LSE_MAX_ABS, ("part LSE", h, r, p)
                assert np.max(np.abs(op[p, 0, r, h] - o_r[0])) <= H.O_MAX_ABS, ("part O", h, r, p)
            o_r, l_r = oracle.head_forward_keys(qrow, kf[:, g], vf[:, g], x.scale, True, q_off, 0, x.Nk)
            assert abs(lg[0, h, r] - l_r[0]) <= H.LSE_MAX_ABS, ("merged LSE", h, r)
            assert np.all(np.abs(og[0, r, h] - o_r[0]) <= H.o_bound(o_r[0])), ("merged O", h, r)


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_split_forced_rescale(tau):
    """Scores rising along the key axis and a late spike inside every chunk: tau 0 and 8 send the
    split kernel's workgroups through the tracking and exact passes; parts and merge match the oracle."""
    B, Nq, Nk, Hq, Hkv, d, n = 1, 200, 900, 4, 2, 128, 3
    x = I.make_split_inputs(B, Nq, Nk, Hq, Hkv, d, True, seed=350, n_splits=n)
    qf = I.bf16_bits_to_f32(x.q)
    kf = I.bf16_bits_to_f32(x.k)
    G = Hq // Hkv
    lean = np.sign(qf.mean(axis=1).reshape(B, Hkv, G, d).mean(axis=2))          # [B, Hkv, d]
    kf = kf + np.linspace(0, 6, Nk, dtype=np.float32)[None, :, None, None] * lean[:, None]
    for j in (250, 550, 880):
        kf[:, j] += 30.0 * lean
    x.k = I.f32_to_bf16_bits(kf)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    opt = capi.FaOptions(capi.FA_EXP_HW, tau, 1)
    o_part, lse_part = ops.forward_split(q, k, v, True, n, x.scale, options=opt)
    o, lse = ops.merge(o_part, lse_part)
    torch.cuda.synchronize()
    op_ref, lp_ref = oracle.attention_forward_split(H.f64(x.q), H.f64(x.k), H.f64(x.v), x.scale, True, n)
    _check_parts(o_part, lse_part, op_ref, lp_ref, f"split forced rescale tau={tau}")
    o_ref, lse_ref = oracle.merge_partials(op_ref, lp_ref)
    H.check_forward(o, lse, o_ref, lse_ref, f"split forced rescale tau={tau} merged")
