"""fa_bwd_noalloc (the backward with its workspace in a fixed device array) against fa_bwd.

Two calls in a row on the same GPU, the second with a smaller problem (and a
packed one after a uniform one), so the second call runs over the array the
first one left behind. Both calls go through the C ABI; their dQ, dK and dV
must equal fa_bwd's bit for bit (the same kernels, deterministic) and meet the
oracle's tolerance.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402

import oracle  # noqa: E402


def _noalloc(x, q, k, v, o, lse, do, cu):
    (dq, bq), (dk, bk), (dv, bv) = (H.poisoned(t.shape, torch.bfloat16) for t in (q, k, v))
    N = x.N
    capi.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, x.B, x.Hq, x.Hkv, N, x.d, int(x.causal), x.scale, cu)
    torch.cuda.synchronize()
    for name, view, buf in (("dQ", dq, bq), ("dK", dk, bk), ("dV", dv, bv)):
        H.assert_fully_written(view, buf, name)
    return dq, dk, dv


def _case(x):
    q, k, v, cu, o, lse = H.gpu_forward(x)
    do = H.dev(x.do)
    ref = ops.backward(q, k, v, o, lse, do, x.causal, x.scale, cu, x.N if cu is not None else None)
    torch.cuda.synchronize()
    got = _noalloc(x, q, k, v, o, lse, do, cu)
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name} differs from fa_bwd"
    rq, rk, rv = oracle.attention_backward(H.f64(x.q), H.f64(x.k), H.f64(x.v), H.f64(x.do), x.scale, x.causal,
                                           x.cu_seqlens)
    for name, g, r in zip(("dQ", "dK", "dV"), got, (rq, rk, rv)):
        e = H.rel_fro(H.host_f64(g), r)
        assert e <= H.GRAD_REL_FRO, f"{name} relative Frobenius error {e:.3e}"


def test_noalloc_matches_fa_bwd_two_calls():
    big = I.make_inputs(2, 700, 8, 2, 128, True, seed=501, with_do=True)
    small = I.make_inputs(1, 129, 4, 4, 64, False, seed=502, with_do=True)
    _case(big)
    _case(small)


def test_noalloc_packed_after_uniform():
    _case(I.make_inputs(1, 520, 4, 2, 128, False, seed=503, with_do=True))
    _case(I.make_inputs(0, 0, 8, 2, 128, True, seed=504, with_do=True, lengths=[300, 1, 0, 129]))


def test_noalloc_rejects_oversized_problem():
    z = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")
    st = capi.fa_bwd_noalloc(z, z, z, z, z, z, z, z, z, 4, 64, 64, 65536, 128, 1, 0.1, None, check=False)
    assert st == capi.FA_ERR_WORKSPACE
