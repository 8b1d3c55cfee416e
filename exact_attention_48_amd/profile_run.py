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
--warm-seconds W   first launch back to back for W seconds, so that the clock has
              settled before the calls that count (select those in a trace with
              ``profile_summary trace --last N``)
--seconds S   launch back to back for S seconds instead of --reps times, and print
              the host-clock time per call
--power       with --seconds: read socket power and the XCDs' gfx clocks from
              ``amd-smi metric`` while the launches run, and print their medians
              (readings of the first second, the clock ramp, are dropped)
Summaries of the profiler's CSV output: ``python -m exact_attention_48_amd.profile_summary``.
Inputs are seeded N(0,1) bf16 drawn on the GPU with the workload's shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import re
import subprocess
import threading
import time

import numpy as np
import torch

from . import capi, inputs as I


def parse_smi_metrics(text: str):
    """(socket power in W, mean gfx clock of the XCDs in MHz) from the JSON of
    ``amd-smi metric --power --clock --json``; None where a reading is missing."""
    vals = []

    def walk(x, path):
        if isinstance(x, dict):
            if "value" in x and "unit" in x:
                vals.append(("/".join(path), x["value"]))
                return
            for k, v in x.items():
                walk(v, path + [str(k)])
        elif isinstance(x, list):
            for i, v in enumerate(x):
                walk(v, path + [str(i)])
    walk(json.loads(text), [])
    pw = [v for k, v in vals if k.endswith("/socket_power") and isinstance(v, (int, float))]
    ck = [v for k, v in vals if re.search(r"/gfx_\d+/clk$", k) and isinstance(v, (int, float))]
    return (float(pw[0]) if pw else None), (sum(ck) / len(ck) if ck else None)


def _power_sampler(stop, samples):
    while not stop.is_set():
        try:
            r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"], capture_output=True, text=True,
                               timeout=10)
            pw, ck = parse_smi_metrics(r.stdout)
        except (OSError, ValueError, subprocess.SubprocessError):
            continue
        if pw is not None and ck is not None:
            samples.append((time.time(), pw, ck))


def _run(launch, args, label):
    if args.warm_seconds > 0:                       # the clock settles over about a second of load
        t0 = time.time()
        n = 0
        while time.time() - t0 < args.warm_seconds:
            launch()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        print(f"{label}: {n} warm-up calls")
    if args.seconds <= 0:
        for _ in range(args.reps):
            launch()
        torch.cuda.synchronize()
        print(f"{label} x {args.reps} done")
        return
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    stop, samples = threading.Event(), []
    th = threading.Thread(target=_power_sampler, args=(stop, samples)) if args.power else None
    t0 = time.time()
    if th:
        th.start()
    n = 0
    while time.time() - t0 < args.seconds:
        for _ in range(4):
            launch()
        n += 4
        torch.cuda.synchronize()
    el = time.time() - t0
    if th:
        stop.set()
        th.join()
    print(f"{label}: {n} calls in {el:.2f} s, {1e3 * el / n:.4f} ms per call (host clock)")
    if args.power:
        late = [x for x in samples if x[0] - t0 >= 1.0]     # past the first second's ramp
        if not late:
            print("power: no amd-smi readings")
            return
        pw = sorted(x[1] for x in late)
        ck = sorted(x[2] for x in late)
        print(f"power: {len(late)} readings after the first second; socket power median {pw[len(pw) // 2]:.0f} W "
              f"(min {pw[0]:.0f}, max {pw[-1]:.0f}); gfx clock, mean of the XCDs, median {ck[len(ck) // 2]:.0f} MHz "
              f"(min {ck[0]:.0f}, max {ck[-1]:.0f})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="fwd_b4_h16_n4096_d128", choices=sorted(I.WORKLOADS))
    ap.add_argument("--part", default="fwd", choices=["fwd", "bwd", "split", "fp8", "copy", "gemm"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--seconds", type=float, default=0.0, help="run back to back for this long instead of --reps")
    ap.add_argument("--power", action="store_true", help="with --seconds: sample amd-smi power and clocks")
    ap.add_argument("--warm-seconds", type=float, default=0.0,
                    help="launch back to back for this long first (untimed; a trace keeps them: see trace --last)")
    ap.add_argument("--exp-mode", type=int, default=capi.FA_EXP_HW, choices=[capi.FA_EXP_HW, capi.FA_EXP_POLY])
    ap.add_argument("--tau", type=float, default=32.0)
    ap.add_argument("--lpt", type=int, default=1, choices=[0, 1])
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    if args.part == "copy":
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        _run(lambda: dst.copy_(src), args, f"copy of {src.numel()} bytes")
        return
    if args.part == "gemm":
        a = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
        _run(lambda: torch.mm(a, b), args, "gemm 8192^3 bf16")
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

        def split_merge():
            capi.fa_fwd_split(q, k, v, op, lp, w.B, w.Hq, w.Hkv, w.N, w.Nk, w.d, int(w.causal), w.scale, w.n_splits)
            capi.fa_merge(op, lp, o, lse, w.n_splits, w.B, w.Hq, w.N, w.d)
        _run(split_merge, args, f"split on {args.workload}")
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
        _run(lambda: capi.fa_fwd_fp8(q8, k8, v, qd, kd, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale),
             args, f"fp8 on {args.workload}")
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
        _run(fwd, args, f"fwd on {args.workload}")
        return
    fwd()
    do = rnd(qs)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = capi.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), int(w.varlen))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _run(lambda: capi.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, w.B, w.Hq, w.Hkv, N, w.d, int(w.causal), w.scale, cu,
                             ws, nb), args, f"bwd on {args.workload}")


if __name__ == "__main__":
    main()
