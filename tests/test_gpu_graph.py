"""The forward and backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a captured forward + backward must replay to the
same bits as the eager calls: on the captured inputs, and again after new input
values are copied into the same buffers. Outputs are NaN-filled eagerly before
every replay, and eager work runs between replays.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


@pytest.mark.parametrize("packed", [False, True], ids=["uniform", "packed"])
def test_graph_replay_matches_eager(packed):
    B, N, Hq, Hkv, d = 2, 300, 4, 2, 128
    if packed:
        lens = [300, 1, 0, 257]
        xs = [I.make_inputs(len(lens), max(lens), Hq, Hkv, d, True, seed=s, with_do=True, lengths=np.array(lens))
              for s in (71, 72)]
    else:
        xs = [I.make_inputs(B, N, Hq, Hkv, d, True, seed=s, with_do=True) for s in (71, 72)]
    x0 = xs[0]
    q, k, v, do = (H.dev(t) for t in (x0.q, x0.k, x0.v, x0.do))
    cu = torch.from_numpy(x0.cu_seqlens).to("cuda:0") if packed else None
    n_max = x0.N if packed else None
    o, lse = torch.empty_like(q), torch.empty(((Hq, q.shape[0]) if packed else (B, Hq, N)), dtype=torch.float32,
                                              device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = capi.fa_bwd_workspace_size(x0.B, Hq, Hkv, x0.N, d, 1, int(packed))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")

    def step():
        ops.forward(q, k, v, True, x0.scale, cu, n_max, out=o, lse=lse)
        ops.backward(q, k, v, o, lse, do, True, x0.scale, cu, n_max, workspace=ws, dq=dq, dk=dk, dv=dv)

    def eager(x):
        for dst, src in zip((q, k, v, do), (x.q, x.k, x.v, x.do)):
            dst.copy_(H.dev(src))
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in (o, lse, dq, dk, dv)]

    refs = [eager(x) for x in xs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device="cuda:0")
    for rep, i in enumerate((0, 1, 0, 1)):
        for dst, src in zip((q, k, v, do), (xs[i].q, xs[i].k, xs[i].v, xs[i].do)):
            dst.copy_(H.dev(src))
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        b = a @ a                           # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(b).all()
        for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), refs[i]):
            assert torch.equal(got, want), f"replay {rep} (inputs {i}): {name} differs from the eager call"
    # and the eager result itself against the oracle, so the replays are checked against it too
    o_ref, lse_ref = H.oracle_forward(xs[1])
    H.check_forward(refs[1][0], refs[1][1], o_ref, lse_ref, "graph inputs 1")
