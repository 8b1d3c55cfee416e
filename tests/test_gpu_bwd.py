"""Backward parity of the HIP kernels (through the C ABI) against the float64 oracle.

The GPU backward consumes the GPU forward's bf16 O and fp32 LSE, as the ABI
prescribes; the oracle recomputes everything from Q, K, V and dO.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def gpu_fwd_bwd(x: I.Inputs):
    q, k, v, cu, o, lse = H.gpu_forward(x)
    do = H.dev(x.do)
    dq, dk, dv = ops.backward(q, k, v, o, lse, do, x.causal, x.scale, cu, x.N if cu is not None else None)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_grads(x: I.Inputs, dq, dk, dv, label):
    rq, rk, rv = oracle.attention_backward(H.f64(x.q), H.f64(x.k), H.f64(x.v), H.f64(x.do), x.scale, x.causal,
                                           x.cu_seqlens)
    errs = []
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        a = H.host_f64(g)
        assert np.all(np.isfinite(a)), f"{label}: non-finite {name}"
        e = H.rel_fro(a, r)
        errs.append(e)
        assert e <= H.GRAD_REL_FRO, f"{label}: {name} relative Frobenius error {e:.3e} > {H.GRAD_REL_FRO}"
    return errs


SMALL = [
    (1, 1, 1, 1, 64, True),
    (2, 7, 2, 2, 64, True),
    (1, 64, 4, 1, 128, False),
    (1, 129, 4, 2, 128, True),
    (2, 200, 2, 1, 64, False),
    (1, 300, 4, 4, 128, True),
    (1, 515, 4, 2, 128, False),
    (1, 300, 256, 256, 128, True),     # the widest K/V rows the library takes (Hkv * d = 32768)
    (1, 200, 512, 256, 64, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full"))
def test_backward_small(case):
    B, N, Hq, Hkv, d, causal = case
    x = I.make_inputs(B, N, Hq, Hkv, d, causal, seed=2000 + N + d, with_do=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, str(case))
    check_grads(x, dq, dk, dv, str(case))


@pytest.mark.parametrize("d", [64, 128])
def test_many_short_sequences(d):
    """A packed batch of 400 sequences of 0-200 tokens (Hq 8, Hkv 2, causal): the
    dK/dV schedule's binary search over a long prefix table, hundreds of ragged
    tile ends, and workgroups that start past their sequence's end. Forward and
    backward against the oracle; every dK/dV row is also checked per sequence."""
    rng = np.random.default_rng(640 + d)
    lens = rng.integers(0, 201, size=400)
    lens[:3] = [0, 1, 200]
    x = I.make_inputs(0, 0, 8, 2, d, True, seed=641 + d, with_do=True, lengths=lens)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"400 sequences d={d}")
    check_grads(x, dq, dk, dv, f"400 sequences d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_zero_scale(causal):
    """softmax_scale = 0: P is uniform over the visible keys, so dV = P^T dO is a
    running mean of dO, while dQ = scale dS K and dK = scale dS^T Q vanish exactly."""
    x = I.make_inputs(2, 300, 4, 2, 128, causal, seed=63, scale=0.0, with_do=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    rq, rk, rv = oracle.attention_backward(H.f64(x.q), H.f64(x.k), H.f64(x.v), H.f64(x.do), x.scale, x.causal)
    assert not np.any(rq) and not np.any(rk)
    assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(dk).item() == 0, "dQ and dK must be exactly 0"
    e = H.rel_fro(H.host_f64(dv), rv)
    assert e <= H.GRAD_REL_FRO, f"dV relative Frobenius error {e:.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_varlen_gqa(causal, d):
    lens = [1, 130, 0, 257, 64, 7, 200]
    x = I.make_inputs(0, 0, 8, 2, d, causal, seed=91 + d, with_do=True, lengths=lens)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    check_grads(x, dq, dk, dv, f"varlen d={d} causal={causal}")


# Packed batches split each (sequence, K/V head)'s tiles over 8 / gcd(Hkv, 8)
# XCDs: 1 way for Hkv = 8, 8 ways for Hkv = 3; the 700-token sequence spans six
# 128-key tiles and three 256-query tiles.
@pytest.mark.parametrize("heads", [(8, 8), (6, 3)], ids=["hq8_hkv8", "hq6_hkv3"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_head_splits(heads, causal):
    Hq, Hkv = heads
    lens = [700, 1, 0, 257, 129, 383]
    x = I.make_inputs(0, 0, Hq, Hkv, 128, causal, seed=95 + Hkv, with_do=True, lengths=lens)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    check_grads(x, dq, dk, dv, f"varlen Hq={Hq} Hkv={Hkv} causal={causal}")


def gpu_fwd_bwd_poisoned(x: I.Inputs):
    """fa_fwd then fa_bwd with dQ/dK/dV written into NaN-filled buffers that carry a NaN
    guard region; asserts that every element was written and nothing past the end."""
    q, k, v, cu, o, lse = H.gpu_forward(x)
    do = H.dev(x.do)
    (dq, bq), (dk, bk), (dv, bv) = (H.poisoned(t.shape, torch.bfloat16) for t in (q, k, v))
    ops.backward(q, k, v, o, lse, do, x.causal, x.scale, cu, x.N if cu is not None else None, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, view, buf in (("dQ", dq, bq), ("dK", dk, bk), ("dV", dv, bv)):
        H.assert_fully_written(view, buf, name)
    return o, lse, dq, dk, dv


def _check_all_heads(x: I.Inputs, dq, dk, dv, label):
    """Every (batch, K/V head) group of a uniform batch against the oracle, one head at a time."""
    q, k, v, do = (H.f64(t) for t in (x.q, x.k, x.v, x.do))
    gq, gk, gv = H.host_f64(dq), H.host_f64(dk), H.host_f64(dv)
    G = x.Hq // x.Hkv
    worst = [0.0, 0.0, 0.0]
    for b in range(x.B):
        for g in range(x.Hkv):
            rk, rv = np.zeros_like(k[b, :, g]), np.zeros_like(v[b, :, g])
            for h in range(g * G, (g + 1) * G):
                rq, hk, hv = oracle.head_backward(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h], x.scale, x.causal)
                rk += hk
                rv += hv
                e = H.rel_fro(gq[b, :, h], rq)
                worst[0] = max(worst[0], e)
                assert e <= H.GRAD_REL_FRO, f"{label} (b={b}, h={h}): dQ relative Frobenius error {e:.3e}"
            for i, (name, a, r) in enumerate((("dK", gk[b, :, g], rk), ("dV", gv[b, :, g], rv))):
                e = H.rel_fro(a, r)
                worst[1 + i] = max(worst[1 + i], e)
                assert e <= H.GRAD_REL_FRO, f"{label} (b={b}, kv={g}): {name} relative Frobenius error {e:.3e}"
    print(f"{label}: worst relative Frobenius errors over all heads dQ {worst[0]:.2e} dK {worst[1]:.2e} "
          f"dV {worst[2]:.2e}")


def test_backward_workload_full_size():
    """bwd_causal_b2_h16_n8192_d128 at full size: all 32 (batch, head) pairs against the oracle,
    outputs NaN-poisoned with guard regions; the sum rules hold on every head as well."""
    x = I.workload_inputs("bwd_causal_b2_h16_n8192_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd_poisoned(x)
    _check_all_heads(x, dq, dk, dv, "bwd_causal_b2_h16_n8192_d128")
    dk2, dv2, do2 = (t.reshape(-1, t.shape[2], t.shape[3]) for t in (dk, dv, H.dev(x.do)))
    segs = [(b * x.N, (b + 1) * x.N) for b in range(x.B)]
    _sum_rules(x, dk2, dv2, do2, segs, "bwd_causal_b2_h16_n8192_d128")


def test_backward_noncausal_full_size():
    """The non-causal B4 Hq16 N4096 d128 backward (the timed step's shape): all 64 (batch, head)
    pairs against the oracle, outputs NaN-poisoned with guard regions."""
    x = I.make_inputs(4, 4096, 16, 16, 128, False, seed=2, with_do=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd_poisoned(x)
    _check_all_heads(x, dq, dk, dv, "bwd_b4_h16_n4096_d128")


def _f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


# Sum rules, per (sequence, K/V head) and column: sum_j dK_j = 0 and sum_j dV_j equals the
# sum over the group's query heads of sum_i dO_i (rows of P sum to one). The kernels round P
# and dS to bf16 before their products (relative 2^-9 per element) and their outputs to bf16,
# so the sums do not vanish exactly. The bounds are set from the residuals measured on the
# causal B2 Hq16 N8192 backward, whose every head the oracle validates (relative Frobenius
# error <= 2.6e-3 there): worst |sum dK| / |dK column| 1.2e-2 and |sum dV - sum dO| / |dV column|
# 8.9e-3 (the packed GQA and 65536-token backward measured 1.4e-2 / 9.1e-3 and 1.1e-2 / 7.9e-3),
# with a margin of 2 to 2.5. The dV rule also allows 2^-9 of |sum dO|; it still rejects a dV
# scaled by 1 + 1 % (checked on every call). The old bounds (5 % of the column norm for dK,
# 2 % of max |sum dO| + 0.5 for dV) passed a 1 % dV scale error.
DK_REL = 2.0 ** -5
DV_REL = 2.0 ** -6


def _sum_rule_residuals(x: I.Inputs, dk, dv, do, a, b):
    G = x.Hq // x.Hkv
    sk = dk[a:b].double().sum(dim=0)                         # [Hkv, d]
    nk = dk[a:b].double().pow(2).sum(dim=0).sqrt()
    sv = dv[a:b].double().sum(dim=0)
    nv = dv[a:b].double().pow(2).sum(dim=0).sqrt()
    so = do[a:b].double().sum(dim=0).reshape(x.Hkv, G, -1).sum(dim=1)
    rk = float((sk.abs() / (nk + 1e-30)).max())
    ok_k = bool((sk.abs() <= DK_REL * nk + 1e-6).all())
    rv = float(((sv - so).abs() / (nv + 1e-30)).max())
    ok_v = bool(((sv - so).abs() <= DV_REL * nv + 2.0 ** -9 * so.abs() + 1e-3).all())
    return rk, rv, ok_k, ok_v


def _sum_rules(x: I.Inputs, dk, dv, do, segments, label):
    """The sum rules on every (sequence, K/V head); sums in float64 on the GPU, any size.
    The check is also run on dV scaled by 1.01, which it must reject."""
    res = [(a, b, *_sum_rule_residuals(x, dk, dv, do, a, b)) for (a, b) in segments]
    worst_k = max(r[2] for r in res)
    worst_v = max(r[3] for r in res)
    print(f"{label}: sum rules, worst |sum dK| / |dK col| {worst_k:.2e} (bound {DK_REL:.2e}), "
          f"|sum dV - sum dO| / |dV col| {worst_v:.2e} (bound {DV_REL:.2e} + 2^-9 |sum dO|)")
    for (a, b, rk, rv, ok_k, ok_v) in res:
        assert ok_k, f"{label}: sum_j dK_j != 0 for tokens {a}..{b} (|sum| / |col| = {rk:.2e})"
        assert ok_v, f"{label}: sum_j dV_j != sum dO for tokens {a}..{b} (|diff| / |col| = {rv:.2e})"
    a, b = max(segments, key=lambda ab: ab[1] - ab[0])
    assert not _sum_rule_residuals(x, dk, dv * 1.01, do, a, b)[3], f"{label}: the dV rule misses a 1 % scale error"


def _check_dq_rows(x: I.Inputs, dq, a, b, heads, label):
    """dQ on the first and last row of every 32-row block of one sequence (tokens a..b)
    against the row-sampled oracle."""
    G = x.Hq // x.Hkv
    rows = H.block_rows()(0, b - a)
    for h in heads:
        g = h // G
        ref = oracle.head_backward_dq_rows(_f64(x.q[a:b, h]), _f64(x.k[a:b, g]), _f64(x.v[a:b, g]),
                                           _f64(x.do[a:b, h]), x.scale, x.causal, rows)
        got = dq[a:b, h][torch.from_numpy(rows).to(dq.device)].double().cpu().numpy()
        e = H.rel_fro(got, ref)
        assert e <= H.GRAD_REL_FRO, f"{label}: dQ rows of head {h}: relative Frobenius error {e:.3e}"


def test_backward_varlen_gqa_full_size():
    """bwd_causal_varlen16_hq32_hkv8_d128 (16 packed sequences of 512..16384 tokens, 4 query heads per
    K/V head): whole K/V groups of the two shortest sequences against the oracle, dQ on the first and
    last row of every 32-row block of the longest one, and the gradient sum rules on every
    (sequence, K/V head); outputs NaN-poisoned with guard regions."""
    x = I.workload_inputs("bwd_causal_varlen16_hq32_hkv8_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd_poisoned(x)
    cu = x.cu_seqlens
    lens = np.diff(cu)
    G = x.Hq // x.Hkv
    for s in np.argsort(lens)[:2]:
        a, b = int(cu[s]), int(cu[s + 1])
        for g in (0, x.Hkv - 1):
            kg, vg = _f64(x.k[a:b, g]), _f64(x.v[a:b, g])
            rk, rv = np.zeros_like(kg), np.zeros_like(vg)
            for h in range(g * G, (g + 1) * G):
                rq, gk, gv = oracle.head_backward(_f64(x.q[a:b, h]), kg, vg, _f64(x.do[a:b, h]), x.scale, True)
                rk += gk
                rv += gv
                e = H.rel_fro(dq[a:b, h].double().cpu().numpy(), rq)
                assert e <= H.GRAD_REL_FRO, f"seq {s} head {h}: dQ relative Frobenius error {e:.3e}"
            for name, got, ref in (("dK", dk[a:b, g], rk), ("dV", dv[a:b, g], rv)):
                e = H.rel_fro(got.double().cpu().numpy(), ref)
                assert e <= H.GRAD_REL_FRO, f"seq {s} K/V head {g}: {name} relative Frobenius error {e:.3e}"
    s = int(np.argmax(lens))
    _check_dq_rows(x, dq, int(cu[s]), int(cu[s + 1]), (0, x.Hq - 1), f"longest sequence {s}")
    do = H.dev(x.do)
    _sum_rules(x, dk, dv, do, [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens)) if lens[i] > 0], "varlen")


def test_backward_long_context():
    """bwd_causal_b1_h8_n65536_d128: dQ on the first and last row of every 32-row block of two heads,
    sum rules on every head; outputs NaN-poisoned with guard regions."""
    x = I.workload_inputs("bwd_causal_b1_h8_n65536_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd_poisoned(x)
    N = x.N
    dq2, dk2, dv2, do2 = (t.reshape(N, t.shape[2], t.shape[3]) for t in (dq, dk, dv, H.dev(x.do)))
    xs = I.Inputs(q=x.q.reshape(N, x.Hq, x.d), k=x.k.reshape(N, x.Hkv, x.d), v=x.v.reshape(N, x.Hkv, x.d),
                  do=x.do.reshape(N, x.Hq, x.d), cu_seqlens=None, B=1, N=N, Hq=x.Hq, Hkv=x.Hkv, d=x.d,
                  causal=x.causal, scale=x.scale)
    _check_dq_rows(xs, dq2, 0, N, (0, x.Hq - 1), "N=65536")
    _sum_rules(xs, dk2, dv2, do2, [(0, N)], "N=65536")


def test_preprocess_rowdot_matches_oracle():
    """The pre-pass alone (fa_bwd_ex with FA_BWD_PREPROCESS) writes -D_i = -sum_k dO_ik O_ik and
    LSE_i log2(e) into the workspace; D against oracle.backward_rowdot of the same bf16 dO and O."""
    x = I.make_inputs(2, 333, 4, 2, 128, True, seed=33, with_do=True)
    q, k, v, cu, o, lse = H.gpu_forward(x)
    do = H.dev(x.do)
    B, N, Hq, Hkv, d = x.B, x.N, x.Hq, x.Hkv, x.d
    nbytes = capi.fa_bwd_workspace_size(B, Hq, Hkv, N, d, 1, 0)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda:0")
    z = torch.empty_like(q)
    capi.fa_bwd_ex(q, k, v, o, lse, do, z, z, z, B, Hq, Hkv, N, d, 1, x.scale, None, ws, nbytes,
                   capi.FA_BWD_PREPROCESS)
    torch.cuda.synchronize()
    half = ((B * N * Hq * 4 + 255) // 256 * 256) // 4
    neg_d = ws[:B * Hq * N].view(B, Hq, N).double().cpu().numpy()
    lse2 = ws[half:half + B * Hq * N].view(B, Hq, N).double().cpu().numpy()
    ref = oracle.backward_rowdot(H.f64(x.do), H.host_f64(o))          # [B, Hq, N]
    assert np.max(np.abs(-neg_d - ref)) <= 1e-4 * (1 + np.max(np.abs(ref)))
    assert np.max(np.abs(lse2 - H.host_f64(lse) * np.log2(np.e))) <= 1e-5 * (1 + np.max(np.abs(lse2)))


def test_backward_deterministic_and_fully_written():
    x = I.make_inputs(1, 300, 4, 2, 128, True, seed=21, with_do=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any()
    _, _, dq2, dk2, dv2 = gpu_fwd_bwd(x)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_workspace_checks():
    z = torch.zeros(64, dtype=torch.bfloat16, device="cuda:0")
    need = capi.fa_bwd_workspace_size(1, 2, 2, 128, 128, 1, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    st = capi.fa_bwd(z, z, z, z, z, z, z, z, z, 1, 2, 2, 128, 128, 1, 0.1, None, ws, need - 1, check=False)
    assert st == capi.FA_ERR_WORKSPACE
    st = capi.fa_bwd(z, z, z, z, z, z, z, z, z, 1, 2, 2, 128, 128, 1, 0.1, None, None, 0, check=False)
    assert st == capi.FA_ERR_WORKSPACE
