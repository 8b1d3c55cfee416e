"""Launch one part of the attention path repeatedly, for hardware-counter runs.

Meant to run under ``rocprofv3 --pmc ...`` (or ``--kernel-trace``):

    python -m exact_attention_48_amd.profile_run --workload fwd_b4_h16_n4096_d128 --part fwd --reps 3

--part fwd    fa_fwd on the workload's shape
--part bwd    fa_fwd once, then fa_bwd `reps` times
--part split  fa_fwd_split (the workload's chunk count) then fa_merge, `reps` times
              (split-KV workloads)
--part fp8    fa_fwd_fp8 `reps` times (8-bit Q/K workloads; E4M3 codes from a
              scaled N(0,1) draw, descale 1/64)
--part copy   a plain device-to-device copy of 512 MiB (known byte count, used
              to calibrate FETCH_SIZE / WRITE_SIZE against real HBM bytes)
--part gemm   torch.mm of two 8192 x 8192 bf16 matrices (the ROCm GEMM library on
              the same matrix cores: clock and MFMA busy of a plain dense GEMM
              beside the attention kernels')
--exp-mode, --tau, --lpt   forward options (fa_fwd_ex) for --part fwd / bwd
Summaries of the profiler's CSV output: ``python -m exact_attention_48_amd.profile_summary``.
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
    ap.add_argument("--part", default="fwd", choices=["fwd", "bwd", "split", "fp8", "copy", "gemm"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--exp-mode", type=int, default=capi.FA_EXP_HW, choices=[capi.FA_EXP_HW, capi.FA_EXP_POLY])
    ap.add_argument("--tau", type=float, default=32.0)
    ap.add_argument("--lpt", type=int, default=1, choices=[0, 1])
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
    if args.part == "gemm":
        a = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
        for _ in range(args.reps):
            torch.mm(a, b)
        torch.cuda.synchronize()
        print(f"gemm 8192^3 bf16 x {args.reps} done")
        return
    w = I.WORKLOADS[args.workload]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    rnd = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    if args.part == "split":
        if w.kind != "split":
            raise SystemExit("--part split needs a split-KV workload")
        q = rnd((w.B, w.N, w.Hq, w.d))
        k, v = rnd((w.B, w.Nk, w.Hkv, w.d)), rnd((w.B, w.Nk, w.Hkv, w.d))
        op = torch.empty((w.n_splits, w.B, w.N, w.Hq, w.d), dtype=torch.float32, device=dev)
        lp = torch.empty((w.n_splits, w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        o = torch.empty((w.B, w.N, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.reps):
            capi.fa_fwd_split(q, k, v, op, lp, w.B, w.Hq, w.Hkv, w.N, w.Nk, w.d, int(w.causal), w.scale, w.n_splits)
            capi.fa_merge(op, lp, o, lse, w.n_splits, w.B, w.Hq, w.N, w.d)
        torch.cuda.synchronize()
        print(f"split x {args.reps} on {args.workload} done")
        return
    if args.part == "fp8":
        if w.kind != "fp8":
            raise SystemExit("--part fp8 needs an 8-bit workload")
        q8 = (rnd((w.B, w.N, w.Hq, w.d)).float() * 64).to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = (rnd((w.B, w.N, w.Hkv, w.d)).float() * 64).to(torch.float8_e4m3fn).view(torch.uint8)
        v = rnd((w.B, w.N, w.Hkv, w.d))
        qd = torch.full((w.B, w.Hq), 1.0 / 64, dtype=torch.float32, device=dev)
        kd = torch.full((w.B, w.Hkv), 1.0 / 64, dtype=torch.float32, device=dev)
        o = torch.empty((w.B, w.N, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.reps):
            capi.fa_fwd_fp8(q8, k8, v, qd, kd, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale)
        torch.cuda.synchronize()
        print(f"fp8 x {args.reps} on {args.workload} done")
        return
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
    q, k, v = rnd(qs), rnd(ks), rnd(ks)
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    opt = capi.FaOptions(args.exp_mode, args.tau, args.lpt)
    fwd = lambda: capi.fa_fwd_ex(q, k, v, o, lse, w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), w.scale, cu, opt)
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
