"""8-bit Q/K forward (OCP E4M3 with per-(sequence, head) descales) on the GPU against the oracle.

The oracle computes the exact attention of the dequantised Q and K with the
bf16 V; the kernel's scores come from 8-bit matrix-core products, exact in
fp32, so the forward's tolerances apply unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_48_amd import capi, inputs as I, ops
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _dev8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda:0")


def _run(x: I.Fp8Inputs, options=None):
    cu = torch.from_numpy(x.cu_seqlens).to("cuda:0") if x.cu_seqlens is not None else None
    o, lse = ops.forward_fp8(_dev8(x.q8), _dev8(x.k8), H.dev(x.v), torch.from_numpy(x.q_descale).cuda(),
                             torch.from_numpy(x.k_descale).cuda(), x.causal, x.scale, cu,
                             x.N if cu is not None else None, options=options)
    torch.cuda.synchronize()
    return o, lse


def _oracle(x: I.Fp8Inputs, rows=None):
    return oracle.attention_forward_fp8(x.q8, x.k8, H.f64(x.v), x.q_descale.astype(np.float64),
                                        x.k_descale.astype(np.float64), x.scale, x.causal, x.cu_seqlens, rows)


@pytest.mark.parametrize("case", [
    (1, 256, 2, 2, False), (2, 300, 4, 2, True), (1, 129, 8, 1, True), (1, 1, 2, 2, True), (2, 520, 4, 4, False),
], ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_{}".format(*c[:4], "causal" if c[4] else "full"))
def test_fp8_forward_small(case):
    B, N, Hq, Hkv, causal = case
    x = I.make_fp8_inputs(B, N, Hq, Hkv, 128, causal, seed=400 + N)
    o, lse = _run(x)
    o_ref, lse_ref = _oracle(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 {case}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_varlen_gqa(causal):
    x = I.make_fp8_inputs(0, 0, 8, 2, 128, causal, seed=410, lengths=[1, 130, 0, 257, 64, 7, 700])
    o, lse = _run(x)
    o_ref, lse_ref = _oracle(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 varlen causal={causal}")


def test_fp8_descales_are_per_sequence_and_head():
    """Distinct descales per (sequence, head): scaling one head's Q descale by 2 equals doubling its scores."""
    x = I.make_fp8_inputs(2, 200, 4, 2, 128, True, seed=420)
    x.q_descale[1, 3] *= 2.0
    x.k_descale[0, 0] *= 0.5
    o, lse = _run(x)
    o_ref, lse_ref = _oracle(x)
    H.check_forward(o, lse, o_ref, lse_ref, "fp8 descales")


def test_fp8_workload_sampled():
    """fp8_fwd_b4_h16_n4096_d128 at full size (the bench's launch): the first and last row of every
    32-row query block of every (batch, head) against the oracle, so every wave of every tile."""
    w = I.WORKLOADS["fp8_fwd_b4_h16_n4096_d128"]
    x = I.workload_inputs(w.name)
    o, lse = _run(x)
    rows = H.block_rows()
    cov = H.wave_coverage(rows(0, x.N), x.N).sum(axis=0)
    print(f"{w.name}: compared rows per wave slot (summed over tiles): {cov.tolist()}")
    o_ref, lse_ref = _oracle(x, rows=rows)
    H.check_forward(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_forced_rescale(tau):
    """Scores rising along the key axis and a late spike: tau 0 and 8 send the 8-bit kernel's
    workgroups through the tracking and exact passes; the result matches the oracle."""
    x = I.make_fp8_inputs(1, 640, 2, 2, 128, False, seed=430)
    k = oracle.e4m3_to_float(x.k8).astype(np.float32) * x.k_descale[0][None, None, :, None]
    q = oracle.e4m3_to_float(x.q8).astype(np.float32) * x.q_descale[0][None, None, :, None]
    k = k + np.linspace(0, 6, 640, dtype=np.float32)[None, :, None, None] * np.sign(q.mean(axis=1, keepdims=True))
    k[:, 600] += 40.0 * np.sign(q[:, 0])
    x.k8, x.k_descale = I._quantize_heads(k, None, 1)
    o_ref, lse_ref = _oracle(x)
    o, lse = _run(x, capi.FaOptions(capi.FA_EXP_HW, tau, 1))
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 forced rescale tau={tau}")


# ---- one descale per 64-token block of each (sequence, head) (fa_fwd_fp8_blockscale) ----

BLOCK_CASES = [(1, 300, 2, 2, False), (2, 300, 4, 2, True), (1, 129, 8, 1, True), (1, 1, 2, 2, True),
               (2, 520, 4, 4, False), (1, 64, 2, 1, True), (1, 65, 2, 1, False)]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_{}".format(*c[:4], "causal" if c[4] else "full"))
def test_fp8_blockscale_small(case):
    """Blocks of Q and K scaled by 2^-u, u in [0, 4], before quantisation: block descales
    differ by up to 16x between neighbouring blocks."""
    B, N, Hq, Hkv, causal = case
    x = I.make_fp8_inputs(B, N, Hq, Hkv, 128, causal, seed=500 + N, block_scale=True, block_gain=4.0)
    assert x.q_descale.shape == (B, Hq, (N + 63) // 64)
    o, lse = _run(x)
    o_ref, lse_ref = _oracle(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 blocks {case}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_blockscale_varlen_gqa(causal):
    x = I.make_fp8_inputs(0, 0, 8, 2, 128, causal, seed=510, lengths=[1, 130, 0, 257, 64, 7, 700],
                          block_scale=True, block_gain=4.0)
    o, lse = _run(x)
    o_ref, lse_ref = _oracle(x)
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 blocks varlen causal={causal}")


def test_fp8_equal_blocks_equal_per_head():
    """Block descales that all equal the per-(sequence, head) ones give bit-identical O and LSE."""
    x = I.make_fp8_inputs(2, 333, 4, 2, 128, True, seed=520)
    o1, l1 = _run(x)
    nb = (x.N + 63) // 64
    x.q_descale = np.repeat(x.q_descale[:, :, None], nb, axis=2)
    x.k_descale = np.repeat(x.k_descale[:, :, None], nb, axis=2)
    o2, l2 = _run(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["fp8_fwd_b4_h16_n4096_d128", "fp8_fwd_causal_b2_h16_n16384_d128"])
def test_fp8_blockscale_workload_sampled(name):
    """The 8-bit workloads at full size with block descales (blocks scaled by 2^-u, u in [0, 3]):
    the first and last row of every 32-row query block of every (batch, head), so every wave of
    every tile, against the oracle."""
    w = I.WORKLOADS[name]
    x = I.make_fp8_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, w.causal, seed=w.seed, block_scale=True, block_gain=3.0)
    o, lse = _run(x)
    rows = H.block_rows()
    o_ref, lse_ref = _oracle(x, rows=rows)
    H.check_forward(o, lse, o_ref, lse_ref, f"{name} blocks")


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_blockscale_forced_rescale(tau):
    """tau 0 and 8 send the block-scaled kernel's workgroups through the tracking and exact
    passes (maxima in scaled units across tiles of different scales); the result matches."""
    x = I.make_fp8_inputs(1, 640, 2, 2, 128, False, seed=530, block_scale=True, block_gain=4.0)
    o_ref, lse_ref = _oracle(x)
    o, lse = _run(x, capi.FaOptions(capi.FA_EXP_HW, tau, 1))
    H.check_forward(o, lse, o_ref, lse_ref, f"fp8 blocks forced rescale tau={tau}")
