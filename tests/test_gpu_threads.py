"""Entry points called concurrently from several host threads, each on its own stream.

The ABI keeps no per-call state (the only shared state is the read-only, once-per-
device address of the no-allocation entry point's array, which is not used here),
so calls from different threads on different streams must give the same bits as
the same calls made one after another.
"""
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi, inputs as I, ops  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


class Job:
    def __init__(self, x):
        self.x = x
        self.q, self.k, self.v, self.do = (H.dev(t) for t in (x.q, x.k, x.v, x.do))
        self.cu = torch.from_numpy(x.cu_seqlens).to("cuda:0") if x.cu_seqlens is not None else None
        self.n_max = x.N if self.cu is not None else None
        self.o = torch.empty_like(self.q)
        lse_shape = (x.Hq, self.q.shape[0]) if self.cu is not None else (x.B, x.Hq, x.N)
        self.lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda:0")
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        nb = capi.fa_bwd_workspace_size(x.B, x.Hq, x.Hkv, x.N, x.d, int(x.causal), int(self.cu is not None))
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")

    def outs(self):
        return (self.o, self.lse, self.dq, self.dk, self.dv)

    def run(self, stream):
        x = self.x
        for t in self.outs():
            t.fill_(float("nan"))
        ops.forward(self.q, self.k, self.v, x.causal, x.scale, self.cu, self.n_max, stream=stream, out=self.o,
                    lse=self.lse)
        ops.backward(self.q, self.k, self.v, self.o, self.lse, self.do, x.causal, x.scale, self.cu, self.n_max,
                     stream=stream, workspace=self.ws, dq=self.dq, dk=self.dk, dv=self.dv)


def test_concurrent_threads_match_sequential_calls():
    xs = [I.make_inputs(2, 700, 8, 2, 128, True, seed=91, with_do=True),
          I.make_inputs(0, 0, 8, 4, 128, True, seed=92, with_do=True, lengths=np.array([513, 1, 0, 300])),
          I.make_inputs(1, 1000, 4, 4, 64, False, seed=93, with_do=True),
          I.make_inputs(3, 257, 16, 16, 128, False, seed=94, with_do=True)]
    ref_jobs = [Job(x) for x in xs]
    for j in ref_jobs:
        j.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    refs = [[t.clone() for t in j.outs()] for j in ref_jobs]

    jobs = [Job(x) for x in xs]
    errors = []
    barrier = threading.Barrier(len(jobs))

    def worker(i):
        try:
            s = torch.cuda.Stream()                  # default priority
            barrier.wait()
            for it in range(6):
                with torch.cuda.stream(s):
                    jobs[i].run(s)
                s.synchronize()
                for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), jobs[i].outs(), refs[i]):
                    if not torch.equal(got, want):
                        errors.append(f"job {i} iteration {it}: {name} differs from the sequential call")
        except Exception as e:                       # reported below, in the main thread
            errors.append(f"job {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, "; ".join(errors[:5])
    # the sequential results themselves against the oracle (first job)
    o_ref, lse_ref = H.oracle_forward(xs[0])
    H.check_forward(refs[0][0], refs[0][1], o_ref, lse_ref, "threads job 0")
