"""Forward parity of the HIP kernels (through the C ABI) against the float64 oracle."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402

SMALL = [
    # (B, N, Hq, Hkv, d, causal)
    (1, 1, 1, 1, 64, False),
    (1, 1, 2, 1, 128, True),
    (2, 7, 2, 2, 64, True),
    (1, 64, 4, 1, 128, False),
    (1, 129, 4, 2, 128, True),
    (2, 300, 2, 1, 64, False),
    (1, 300, 4, 4, 128, True),
    (1, 383, 2, 2, 64, True),
    (1, 515, 8, 2, 128, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full"))
def test_forward_small(case):
    B, N, Hq, Hkv, d, causal = case
    x = I.make_inputs(B, N, Hq, Hkv, d, causal, seed=1000 + N + d)
    *_, o, lse = H.gpu_forward(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, str(case))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_varlen_gqa(causal, d):
    lens = [1, 130, 0, 257, 64, 7, 200]
    x = I.make_inputs(0, 0, 8, 2, d, causal, seed=77 + d, lengths=lens)
    *_, o, lse = H.gpu_forward(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"varlen d={d} causal={causal}")


# Packed batches split each (sequence, K/V head)'s query tiles over
# 8 / gcd(Hkv, 8) XCDs (1 way for Hkv = 8, 8 ways for Hkv = 3).
@pytest.mark.parametrize("heads", [(8, 8), (6, 3)], ids=["hq8_hkv8", "hq6_hkv3"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_varlen_head_splits(heads, causal):
    Hq, Hkv = heads
    lens = [700, 1, 0, 257, 129, 383]
    x = I.make_inputs(0, 0, Hq, Hkv, 128, causal, seed=81 + Hkv, lengths=lens)
    *_, o, lse = H.gpu_forward(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"varlen Hq={Hq} Hkv={Hkv} causal={causal}")


def test_forward_workload_small_d64():
    """fwd_b1_h2_n256_d64, all rows."""
    x = I.workload_inputs("fwd_b1_h2_n256_d64")
    *_, o, lse = H.gpu_forward(x)
    o_ref, lse_ref = H.oracle_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, "fwd_b1_h2_n256_d64")


@pytest.mark.parametrize("name", ["fwd_b4_h16_n4096_d128", "fwd_causal_b2_h16_n16384_d128",
                                  "fwd_causal_varlen16_hq32_hkv8_d128", "fwd_causal_b1_h16_n131072_d128"])
def test_forward_workload_sampled(name):
    """Full-size workloads with the launch the bench times, checked on every (sequence, head) at
    the first and last row of every 32-row query block, so that every wave of every query
    tile is compared (the per-wave-slot counts are printed and asserted)."""
    x = I.workload_inputs(name)
    *_, o, lse = H.gpu_forward(x)
    rows = H.block_rows()
    lens = np.diff(x.cu_seqlens) if x.cu_seqlens is not None else [x.N] * x.B
    cov = sum(H.wave_coverage(rows(0, int(L)), int(L)).sum(axis=0) for L in lens if L > 0)
    print(f"{name}: compared rows per wave slot (summed over tiles and sequences): {cov.tolist()}")
    o_ref, lse_ref = H.oracle_forward(x, rows=rows)
    H.check_forward(o, lse, o_ref, lse_ref, name)


def test_options_give_same_result():
    """Conditional-rescale threshold, exp mode and tile order do not change the result.
    tau 0 and 8 send the workgroups through the tracking and exact passes, 32 does not."""
    x = I.make_inputs(1, 700, 4, 2, 128, True, seed=5)
    o_ref, lse_ref = H.oracle_forward(x)
    base = None
    for exp_mode in (capi.FA_EXP_HW, capi.FA_EXP_POLY):
        for tau in (0.0, 8.0, 32.0):
            for lpt in (0, 1):
                opt = capi.FaOptions(exp_mode, tau, lpt)
                *_, o, lse = H.gpu_forward(x, opt)
                H.check_forward(o, lse, o_ref, lse_ref, f"exp={exp_mode} tau={tau} lpt={lpt}")
                if exp_mode == capi.FA_EXP_HW and tau == 8.0:
                    if base is None:
                        base = (o.clone(), lse.clone())
                    else:   # tile order must not change a single bit
                        assert torch.equal(o, base[0]) and torch.equal(lse, base[1])


def test_rescale_events_forced():
    """Scores that rise along the key axis and a late spike force many rescales."""
    B, N, NH, d = 1, 640, 2, 128
    x = I.make_inputs(B, N, NH, NH, d, False, seed=9)
    kf = I.bf16_bits_to_f32(x.k).reshape(B, N, NH, d)
    qf = I.bf16_bits_to_f32(x.q).reshape(B, N, NH, d)
    ramp = np.linspace(0, 6, N, dtype=np.float32)[None, :, None, None]
    kf = kf + ramp * np.sign(qf.mean(axis=1, keepdims=True))
    kf[:, 600] += 40.0 * np.sign(qf[:, 0:1, :, :])[:, 0]
    x.k = I.f32_to_bf16_bits(kf)
    o_ref, lse_ref = H.oracle_forward(x)
    # the spike outgrows the first tile's max by far more than the default
    # tau, so every setting takes the exact re-run
    for opt in (None, capi.FaOptions(capi.FA_EXP_HW, 0.0, 1), capi.FaOptions(capi.FA_EXP_HW, 8.0, 1),
                capi.FaOptions(capi.FA_EXP_POLY, 32.0, 1), capi.FaOptions(capi.FA_EXP_POLY, 8.0, 0)):
        *_, o, lse = H.gpu_forward(x, opt)
        label = "default" if opt is None else f"exp={opt.exp_mode} tau={opt.rescale_tau}"
        H.check_forward(o, lse, o_ref, lse_ref, f"ramp {label}")


@pytest.mark.parametrize("exp_mode", [0, 1], ids=["hw", "poly"])
def test_late_score_far_above_first_max(exp_mode):
    """One key of the last tile scores about 450 (650 in log2 units above the first tile's max):
    the polynomial exponential must overflow to +inf there (not wrap to a tiny value), so
    that the row takes the exact re-run in both exponential modes."""
    B, N, NH, d = 1, 300, 2, 128
    x = I.make_inputs(B, N, NH, NH, d, False, seed=19)
    qf = I.bf16_bits_to_f32(x.q).reshape(B, N, NH, d) + 1.0     # every query leans towards (1, ..., 1)
    kf = I.bf16_bits_to_f32(x.k).reshape(B, N, NH, d)
    kf[:, 290] = 40.0                                           # key 290 scores about 450 for every query
    x.q = I.f32_to_bf16_bits(qf)
    x.k = I.f32_to_bf16_bits(kf)
    o_ref, lse_ref = H.oracle_forward(x)
    assert float(np.max(lse_ref)) > 150.0
    *_, o, lse = H.gpu_forward(x, capi.FaOptions(exp_mode, 32.0, 1))
    H.check_forward(o, lse, o_ref, lse_ref, f"late score exp={exp_mode}")


def test_large_scores_stay_finite():
    x = I.make_inputs(1, 256, 2, 2, 128, True, seed=3)
    q = I.bf16_bits_to_f32(x.q) * 100.0
    x.q = I.f32_to_bf16_bits(q)
    o_ref, lse_ref = H.oracle_forward(x)
    *_, o, lse = H.gpu_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, "Q x 100")


def test_deterministic_and_fully_written():
    x = I.make_inputs(2, 333, 4, 2, 128, True, seed=11)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    guard = 4096
    ob = torch.full((q.numel() + guard,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    lb = torch.full((2 * 4 * 333 + guard,), float("nan"), dtype=torch.float32, device="cuda:0")
    o = ob[: q.numel()].view(q.shape)
    lse = lb[: 2 * 4 * 333].view(2, 4, 333)
    ops.forward(q, k, v, True, x.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any(), "some output element was not written"
    assert torch.isnan(ob[q.numel():]).all() and torch.isnan(lb[2 * 4 * 333:]).all(), "write past the end"
    o2, lse2 = ops.forward(q, k, v, True, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_empty_problems_are_noops():
    z = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    assert capi.fa_fwd(z, z, z, z, z, 0, 2, 2, 128, 128, 1, 0.1) == capi.FA_OK
    assert capi.fa_fwd(z, z, z, z, z, 3, 2, 2, 0, 128, 1, 0.1) == capi.FA_OK


@pytest.mark.parametrize("exp_mode", [0, 1], ids=["hw", "poly"])
def test_nan_input_propagates(exp_mode):
    x = I.make_inputs(1, 64, 1, 1, 64, False, seed=2)
    qf = I.bf16_bits_to_f32(x.q)
    qf[0, 5, 0, 3] = np.nan
    x.q = I.f32_to_bf16_bits(qf)
    *_, o, lse = H.gpu_forward(x, capi.FaOptions(exp_mode, 32.0, 1))
    o = H.host_f64(o)
    assert np.all(np.isnan(o[0, 5, 0])), "a NaN query must give a NaN output row"
    assert np.all(np.isfinite(np.delete(o[0, :, 0], 5, axis=0))), "other rows stay finite"


def test_ops_reject_mismatched_tensors():
    """The tensor-level helpers check every tensor's shape before a pointer reaches the C ABI."""
    q = torch.zeros((1, 64, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    v_bad = torch.zeros((1, 32, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        ops.forward(q, k, v_bad, False)
    with pytest.raises(ValueError):
        ops.forward(q, k, k, False, lse=torch.zeros((1, 4, 63), dtype=torch.float32, device="cuda:0"))
    with pytest.raises(ValueError):
        ops.forward(q, k, k, False, out=torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda:0"))
    o, lse = ops.forward(q, k, k, False)
    with pytest.raises(ValueError):
        ops.backward(q, k, k, o[:, :32].contiguous(), lse, o, False)
    with pytest.raises(ValueError):
        ops.backward(q, k, k, o, lse[:, :2].contiguous(), o, False)
    cu = torch.tensor([0, 30, 64], dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):   # packed K with another token count than Q
        ops.forward(q[0], k[0, :60], k[0, :60], True, cu_seqlens=cu, max_seqlen=34)


def test_negative_scale_is_rejected():
    x = I.make_inputs(1, 64, 2, 2, 128, False, seed=4)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    with pytest.raises(capi.FaError):
        ops.forward(q, k, v, False, -0.1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_uniform_weights(d, causal):
    """Scale 0: every visible key gets the same weight, masked keys none (O = mean of the visible
    V rows, LSE = ln of their count); no NaN from a masked score times a zero scale."""
    x = I.make_inputs(1, 300, 2, 2, d, causal, seed=6, scale=0.0)
    o_ref, lse_ref = H.oracle_forward(x)
    *_, o, lse = H.gpu_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"scale 0 d={d} causal={causal}")
    n_vis = np.arange(1, 301) if causal else np.full(300, 300)
    np.testing.assert_allclose(H.host_f64(lse)[0, 0], np.log(n_vis), atol=1e-3)
    # the packed layout with grouped heads, empty and one-token sequences
    x = I.make_inputs(0, 0, 4, 2, d, causal, seed=62, scale=0.0, lengths=np.array([1, 257, 0, 64]))
    o_ref, lse_ref = H.oracle_forward(x)
    *_, o, lse = H.gpu_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"scale 0 packed d={d} causal={causal}")
    lse_h = H.host_f64(lse)
    for a, b in zip(x.cu_seqlens[:-1], x.cu_seqlens[1:]):
        n_vis = np.arange(1, b - a + 1) if causal else np.full(b - a, b - a)
        np.testing.assert_allclose(lse_h[:, a:b], np.broadcast_to(np.log(n_vis), (4, b - a)), atol=1e-3)
