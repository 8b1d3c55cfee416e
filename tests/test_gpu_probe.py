"""The atomic-traffic probe adds what the fused-dQ design would add (counts checked exactly)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import probe  # noqa: E402


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 300, 128), (2, 3, 513, 64)])
def test_dq_atomics_counts(B, H, N, d, causal):
    acc = torch.zeros((B, N, H, d), dtype=torch.float32, device="cuda:0")
    probe.dq_atomics(acc, B, H, N, d, causal)
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    n_kt = (N + 127) // 128
    q = np.arange(N)
    # key tile kt (keys 128 kt ..) adds to every row of the 64-row query tiles from
    # kt * 128 / 64 on (causal) or to every row (non-causal)
    want = np.array([sum(1 for kt in range(n_kt) if not causal or (2 * kt) <= qi // 64) for qi in q], np.float32)
    assert np.array_equal(got, np.broadcast_to(want[None, :, None, None], got.shape))
