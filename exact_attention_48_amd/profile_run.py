"""Launch one part of the attention path repeatedly, for hardware-counter runs.

Meant to run under ``rocprofv3 --pmc ...`` (or ``--kernel-trace``):

    python -m exact_attention_48_amd.profile_run --workload fwd_b4_h16_n4096_d128 --part fwd --reps 3

--part fwd    fa_fwd on the workload's shape
--part bwd    fa_fwd once, then fa_bwd `reps` times
--part copy   a plain device-to-device copy of 512 MiB (known byte count, used
              to calibrate FETCH_SIZE / WRITE_SIZE against real HBM bytes)
Inputs are seeded N(0,1) bf16 drawn on the GPU with the workload's shapes.
"""
from __future__ import annotations

import argparse
import math

import numpy as np
import torch

from . import capi, inputs as I


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="fwd_b4_h16_n4096_d128", choices=sorted(I.WORKLOADS))
    ap.add_argument("--part", default="fwd", choices=["fwd", "bwd", "copy"])
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    if args.part == "copy":
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {src.numel()} bytes x {args.reps}")
        return
    w = I.WORKLOADS[args.workload]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    if w.varlen:
        lens = I.draw_lengths(np.random.default_rng(w.seed), w.B, w.len_lo, w.len_hi)
        cu_h = np.zeros(len(lens) + 1, dtype=np.int32)
        cu_h[1:] = np.cumsum(lens)
        T, N = int(cu_h[-1]), int(lens.max())
        qs, ks, lse_shape = (T, w.Hq, w.d), (T, w.Hkv, w.d), (w.Hq, T)
        cu = torch.from_numpy(cu_h).to(dev)
    else:
        N = w.N
        qs, ks, lse_shape = (w.B, N, w.Hq, w.d), (w.B, N, w.Hkv, w.d), (w.B, w.Hq, N)
        cu = None
    rnd = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q, k, v = rnd(qs), rnd(ks), rnd(ks)
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    fwd = lambda: capi.fa_fwd(q, k, v, o, lse, w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), w.scale, cu)
    if args.part == "fwd":
        for _ in range(args.reps):
            fwd()
    else:
        fwd()
        do = rnd(qs)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nb = capi.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), int(w.varlen))
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(args.reps):
            capi.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), w.scale, cu,
                        ws, nb)
    torch.cuda.synchronize()
    print(f"{args.part} x {args.reps} on {args.workload} done")


if __name__ == "__main__":
    main()
