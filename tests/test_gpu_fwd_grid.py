"""Forward parity on uniform d = 128 batches with more work items (query tiles of
256 rows) than the GPU has CUs, so that every CU runs several of them one after
another: 288-768 items with GQA, causal and non-causal masks, ragged sequence
ends, the widest K/V rows the library takes (256 heads of d = 128) and the
conditional-rescale re-run. Rows checked: the first and last of
every wave's 32 rows in every 256-row tile, plus a stride through the rest.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


def wave_rows(s, L):
    """Row selector: rows 0 and 31 of every wave's 32-row block, every 37th row and the last."""
    rows = {t + w * 32 + r for t in range(0, L, 256) for w in range(8) for r in (0, 31)}
    rows |= set(range(0, L, 37))
    rows |= {L - 1}
    return np.array(sorted(r for r in rows if r < L), dtype=np.int64)


CASES = [
    # B, N, Hq, Hkv, causal: key tiles of 64 per item
    (2, 1000, 40, 40, False),   # 16
    (2, 1000, 40, 10, True),    # 4, 8, 12, 16
    (3, 700, 32, 8, False),     # 11
    (3, 700, 32, 32, True),     # 4, 8, 11
    (1, 700, 256, 256, True),   # the widest K/V rows the library takes (Hkv * d = 32768)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_N{}_Hq{}_Hkv{}_{}".format(*c[:4], "causal" if c[4] else "full"))
def test_forward_many_items(case):
    B, N, Hq, Hkv, causal = case
    assert B * Hq * ((N + 255) // 256) > 256
    x = I.make_inputs(B, N, Hq, Hkv, 128, causal, seed=3000 + N + Hq)
    o_ref, lse_ref = H.oracle_forward(x, rows=wave_rows)
    *_, o, lse = H.gpu_forward(x)
    H.check_forward(o, lse, o_ref, lse_ref, str(case))


def test_forward_many_items_rescale_rerun():
    """Keys that ramp up along the sequence plus a late spike: every work item of
    this 320-item shape takes the tracking and exact re-run passes (tau = 0 and
    the default)."""
    B, N, NH, d = 2, 1000, 40, 128
    x = I.make_inputs(B, N, NH, NH, d, False, seed=3901)
    kf = I.bf16_bits_to_f32(x.k).reshape(B, N, NH, d)
    qf = I.bf16_bits_to_f32(x.q).reshape(B, N, NH, d)
    ramp = np.linspace(0, 6, N, dtype=np.float32)[None, :, None, None]
    kf = kf + ramp * np.sign(qf.mean(axis=1, keepdims=True))
    kf[:, 900] += 40.0 * np.sign(qf[:, 0:1, :, :])[:, 0]
    x.k = I.f32_to_bf16_bits(kf)
    o_ref, lse_ref = H.oracle_forward(x, rows=wave_rows)
    for opt in (None, capi.FaOptions(capi.FA_EXP_HW, 0.0, 1)):
        *_, o, lse = H.gpu_forward(x, opt)
        H.check_forward(o, lse, o_ref, lse_ref, "re-run " + ("default" if opt is None else "tau=0"))


def test_forward_many_items_fully_written_and_deterministic():
    B, N, Hq, Hkv = 3, 700, 32, 8
    x = I.make_inputs(B, N, Hq, Hkv, 128, True, seed=3902)
    q, k, v = H.dev(x.q), H.dev(x.k), H.dev(x.v)
    guard = 4096
    ob = torch.full((q.numel() + guard,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    lb = torch.full((B * Hq * N + guard,), float("nan"), dtype=torch.float32, device="cuda:0")
    o = ob[: q.numel()].view(q.shape)
    lse = lb[: B * Hq * N].view(B, Hq, N)
    ops.forward(q, k, v, True, x.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any(), "some output element was not written"
    assert torch.isnan(ob[q.numel():]).all() and torch.isnan(lb[B * Hq * N:]).all(), "write past the end"
    o2, lse2 = ops.forward(q, k, v, True, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
