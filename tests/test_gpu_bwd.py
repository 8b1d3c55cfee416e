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
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full"))
def test_backward_small(case):
    B, N, Hq, Hkv, d, causal = case
    x = I.make_inputs(B, N, Hq, Hkv, d, causal, seed=2000 + N + d, with_do=True)
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, str(case))
    check_grads(x, dq, dk, dv, str(case))


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


def test_backward_workload_full_size():
    """bwd_causal_b2_h16_n8192_d128: two whole heads against the oracle, invariants on all heads."""
    x = I.workload_inputs("bwd_causal_b2_h16_n8192_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    q, k, v, do = (H.f64(t) for t in (x.q, x.k, x.v, x.do))
    gq, gk, gv = H.host_f64(dq), H.host_f64(dk), H.host_f64(dv)
    for (b, h) in ((0, 0), (1, 15)):
        rq, rk, rv = oracle.head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], x.scale, True)
        for name, a, r in (("dQ", gq[b, :, h], rq), ("dK", gk[b, :, h], rk), ("dV", gv[b, :, h], rv)):
            e = H.rel_fro(a, r)
            assert e <= H.GRAD_REL_FRO, f"(b={b}, h={h}) {name} relative Frobenius error {e:.3e}"
    # oracle-free invariants on every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    sk = gk.sum(axis=1)
    assert np.all(np.abs(sk) <= 0.05 * np.sqrt((gk ** 2).sum(axis=1)) + 1e-3)
    sv, so = gv.sum(axis=1), do.sum(axis=1)
    assert np.max(np.abs(sv - so)) <= 0.02 * np.max(np.abs(so)) + 0.5


def _f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def _sum_rules(x: I.Inputs, dk, dv, do, segments, label):
    """Per (sequence, K/V head): sum_j dK_j = 0 and sum_j dV_j = sum over the group's query
    heads of sum_i dO_i (rows of P sum to one). Sums in float64 on the GPU; any size."""
    G = x.Hq // x.Hkv
    for (a, b) in segments:
        sk = dk[a:b].double().sum(dim=0)                         # [Hkv, d]
        nk = dk[a:b].double().pow(2).sum(dim=0).sqrt()
        sv = dv[a:b].double().sum(dim=0)
        so = do[a:b].double().sum(dim=0).reshape(x.Hkv, G, -1).sum(dim=1)
        assert bool((sk.abs() <= 0.05 * nk + 1e-3).all()), f"{label}: sum_j dK_j != 0 for tokens {a}..{b}"
        assert float((sv - so).abs().max()) <= 0.02 * float(so.abs().max()) + 0.5, f"{label}: sum dV != sum dO"


def _check_dq_rows(x: I.Inputs, dq, a, b, heads, label):
    """dQ on sampled rows of one sequence (tokens a..b) against the row-sampled oracle."""
    G = x.Hq // x.Hkv
    rows = H.sampled_rows(n_first=64, n_last=64, stride=509)(0, b - a)
    for h in heads:
        g = h // G
        ref = oracle.head_backward_dq_rows(_f64(x.q[a:b, h]), _f64(x.k[a:b, g]), _f64(x.v[a:b, g]),
                                           _f64(x.do[a:b, h]), x.scale, x.causal, rows)
        got = dq[a:b, h][torch.from_numpy(rows).to(dq.device)].double().cpu().numpy()
        e = H.rel_fro(got, ref)
        assert e <= H.GRAD_REL_FRO, f"{label}: dQ rows of head {h}: relative Frobenius error {e:.3e}"


def test_backward_varlen_gqa_full_size():
    """bwd_causal_varlen16_hq32_hkv8_d128 (16 packed sequences of 512..16384 tokens, 4 query heads per
    K/V head): whole K/V groups of the two shortest sequences against the oracle, dQ on sampled rows of
    the longest one, and the gradient sum rules on every (sequence, K/V head)."""
    x = I.workload_inputs("bwd_causal_varlen16_hq32_hkv8_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
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
    """bwd_causal_b1_h8_n65536_d128: dQ on sampled rows of two heads, sum rules on every head."""
    x = I.workload_inputs("bwd_causal_b1_h8_n65536_d128")
    o, lse, dq, dk, dv = gpu_fwd_bwd(x)
    N = x.N
    dq2, dk2, dv2, do2 = (t.reshape(N, t.shape[2], t.shape[3]) for t in (dq, dk, dv, H.dev(x.do)))
    xs = I.Inputs(q=x.q.reshape(N, x.Hq, x.d), k=x.k.reshape(N, x.Hkv, x.d), v=x.v.reshape(N, x.Hkv, x.d),
                  do=x.do.reshape(N, x.Hq, x.d), cu_seqlens=None, B=1, N=N, Hq=x.Hq, Hkv=x.Hkv, d=x.d,
                  causal=x.causal, scale=x.scale)
    _check_dq_rows(xs, dq2, 0, N, (0, x.Hq - 1), "N=65536")
    _sum_rules(xs, dk2, dv2, do2, [(0, N)], "N=65536")


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
