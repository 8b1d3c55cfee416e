#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd: D pre-pass, dK/dV
kernel, dQ kernel) over one batch of the B=4, Hq=Hkv=16, N=4096, d=128,
non-causal workload, inputs resident in HBM. Counted work per step follows
the FLOP convention of the metric: 4*B*Hq*N^2*d for the forward (halved for
causal) and 2.5x that for the backward.

Prints ONE JSON line with the step throughput (TFLOP/s), the roofline of the
dominant kernel (timed live with HIP events on its launch stream), per-kernel
and per-workload figures, and the float64 CPU oracle timed on a bounded sample
on this machine's host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--main-only]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_48_amd.kernel_sources import source_hash  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz (AMD: "2.5 PFLOP/s" dense BF16)
PEAK_FP8_TFLOPS = 5033.2      # dense 8-bit MFMA, twice the bf16 rate (AMD: "5.0 PFLOP/s")
# the 8-bit Q/K forward runs half its counted work (Q K^T) at the 8-bit rate and half (P V) at the bf16 rate
PEAK_QK8_PV16_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X (% of dense BF16 MFMA peak)"
MAIN = "fwd_b4_h16_n4096_d128"

# Algorithmic work of each kernel per unmasked score element, in units of d FLOP:
# forward: S = QK^T and O = PV (4d); dK/dV kernel: S, dP, dV, dK (8d); dQ kernel:
# the dQ product only (2d; its S and dP recomputations are not algorithmic).
# (d = 128 forwards run fa_fwd_pp_kernel, the two-waves-per-SIMD kernel; other d run fa_fwd_kernel)
FWD_OPTION_TIMINGS = {}
# The workload on which the dQ options are timed side by side (the causal 8192-token backward).
DQ_AB_WORKLOAD = "bwd_causal_b2_h16_n8192_d128"
KERNEL_FLOP_PER_ELEM = {"fa_fwd_pp_kernel": 4, "fa_fwd_kernel": 4, "bwd_dkdv_kernel": 8, "bwd_dq_kernel": 2,
                        "bwd_prep_kernel": 0}


# Forward timings under non-default options, beside the default (v_exp_f32, tau = 32,
# heaviest tiles first): the software exponential, the plain tile order, and tau = 0,
# which sends every workgroup through the tracking and exact re-run passes (the cost
# of the conditional-rescale fallback when it fires everywhere).
def _fwd_option_timings():
    from exact_attention_48_amd import capi
    poly = ("exp_poly", capi.FaOptions(capi.FA_EXP_POLY, 32.0, 1))
    lpt0 = ("lpt0", capi.FaOptions(capi.FA_EXP_HW, 32.0, 0))
    tau0 = ("tau0_rerun", capi.FaOptions(capi.FA_EXP_HW, 0.0, 1))
    return {"fwd_b4_h16_n4096_d128": [poly, tau0], "fwd_causal_b2_h16_n16384_d128": [poly, lpt0, tau0],
            "fwd_causal_varlen16_hq32_hkv8_d128": [lpt0]}


def steady_ms(fn, reps, stream, warm_s=1.0):
    """Milliseconds per call in steady state: back-to-back calls for warm_s seconds first
    (after an idle gap the clock takes about a second to settle: the first window runs
    ~10 % slow and the next ones 1.5-2.5 % slow), then the median of five timed windows
    of `reps` calls, timed with HIP events on `stream`."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    windows = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        windows.append(a.elapsed_time(b) / reps)
    return sorted(windows)[2]


def library_reference():
    """What the ROCm libraries reach on this device under the same clock and power
    limits: a large bf16 GEMM through torch.mm (hipBLASLt), the practical matrix-core
    ceiling, and torch's fused attention (flash backend only, never the math path) on
    the two d = 128 forward workloads. Context for the kernels' fractions, not inputs.
    Runs in a child process of the benchmark, so that a failure here cannot cost the
    benchmark its own line."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import sdpa_kernel, SDPBackend
    from exact_attention_48_amd import inputs as I
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev)
    out = {}
    M = 8192
    g.manual_seed(1)
    a_m = torch.randn(M, M, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b_m = torch.randn(M, M, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ms = steady_ms(lambda: torch.mm(a_m, b_m), 10, stream)
    fl = 2.0 * M ** 3
    out["torch_mm_bf16_8192"] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                                 "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del a_m, b_m
    for name in ("fwd_b4_h16_n4096_d128", "fwd_causal_b2_h16_n16384_d128"):
        wl = I.WORKLOADS[name]
        qs = (wl.B, wl.N, wl.Hq, wl.d)
        g.manual_seed(2)
        qt, kt, vt = (torch.randn(qs, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16).transpose(1, 2)
                      for _ in range(3))
        fl = I.counted_flops([wl.N] * wl.B, wl.Hq, wl.d, wl.causal)
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                ms = steady_ms(lambda: F.scaled_dot_product_attention(qt, kt, vt, is_causal=wl.causal,
                                                                      scale=wl.scale), 5, stream)
            out["torch_sdpa_flash_" + name] = {
                "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        except RuntimeError as e:          # no flash kernel for this device in this torch build
            out["torch_sdpa_flash_" + name] = {"unavailable": str(e)[:200]}
        del qt, kt, vt
    return out


def _library_reference_child():
    """The library reference block from a child process (bench.py --library-reference)."""
    import subprocess
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--library-reference"], capture_output=True,
                           text=True, timeout=240)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            return {"unavailable": f"child exited with status {r.returncode}: {r.stderr.strip()[-200:]}"}
        return json.loads(lines[-1])
    except (subprocess.SubprocessError, OSError, ValueError) as e:
        return {"unavailable": repr(e)[:200]}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=500)   # ~1 s: the clock settles before the timed steps
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--main-only", action="store_true", help="skip the per-workload figures")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU-oracle sample (0 = auto)")
    ap.add_argument("--library-reference", action="store_true",
                    help="print only the ROCm library reference figures (one JSON object) and exit")
    return ap.parse_args()


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.library_reference:
        print(json.dumps(library_reference()))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from exact_attention_48_amd import capi, inputs as I, probe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    capi.load()
    dev = torch.device("cuda:0")
    global FWD_OPTION_TIMINGS
    FWD_OPTION_TIMINGS = _fwd_option_timings()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- main workload: one step = fa_fwd + fa_bwd ----------------
    w = I.WORKLOADS[MAIN]
    x = I.make_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, w.causal, w.seed, scale=w.scale, with_do=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    B, N, Hq, Hkv, d, causal, scale = x.B, x.N, x.Hq, x.Hkv, x.d, int(x.causal), x.scale
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = capi.fa_bwd_workspace_size(B, Hq, Hkv, N, d, causal, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def launch_all(evs=None):
        if evs: evs[0].record(stream)
        capi.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, None, stream)
        if evs: evs[1].record(stream)
        capi.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, None, ws, ws_bytes,
                       capi.FA_BWD_PREPROCESS, stream)
        if evs: evs[2].record(stream)
        capi.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, None, ws, ws_bytes,
                       capi.FA_BWD_DKDV, stream)
        if evs: evs[3].record(stream)
        capi.fa_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, None, ws, ws_bytes,
                       capi.FA_BWD_DQ, stream)
        if evs: evs[4].record(stream)

    for _ in range(args.warmup):
        launch_all()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        launch_all(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    names = ["fa_fwd_pp_kernel" if d == 128 else "fa_fwd_kernel", "bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]
    kms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all(), "non-finite outputs"

    lengths = [N] * B
    f_fwd = I.counted_flops(lengths, Hq, d, bool(causal))
    f_bwd = I.counted_flops(lengths, Hq, d, bool(causal), backward=True)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    elems = B * Hq * float(N) * N * (0.5 if causal else 1.0)

    kernels = {}
    for n in names:
        fl = KERNEL_FLOP_PER_ELEM[n] * d * elems
        ent = {"ms": round(kms[n], 4)}
        if fl > 0:
            tf = fl / (kms[n] * 1e-3) / 1e12
            ent.update({"algorithmic_tflop": round(fl / 1e12, 4), "tflops": round(tf, 1),
                        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        else:
            by = B * N * Hq * (2 * d * 2 + 4)
            ent.update({"algorithmic_bytes": by, "gbs": round(by / (kms[n] * 1e-3) / 1e9, 1)})
        kernels[n] = ent
    dom = max(names, key=lambda n: kms[n])
    dom_fl = KERNEL_FLOP_PER_ELEM[dom] * d * elems
    achieved = dom_fl / (kms[dom] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(dom, MAIN)}

    # ---------------- per-workload figures (parity-test shapes) ----------------
    workloads = {}
    if not args.main_only:
        g = torch.Generator(device=dev)

        def rnd(shape, seed):
            g.manual_seed(seed)
            return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

        def time_it(fn, reps):
            return steady_ms(fn, reps, stream)

        for name in ("fwd_b4_h16_n4096_d128", "fwd_causal_b2_h16_n16384_d128",
                     "fwd_causal_varlen16_hq32_hkv8_d128", "bwd_causal_b2_h16_n8192_d128", "fwd_b1_h2_n256_d64",
                     "bwd_causal_varlen16_hq32_hkv8_d128", "fwd_causal_b1_h16_n131072_d128",
                     "bwd_causal_b1_h8_n65536_d128"):
            wl = I.WORKLOADS[name]
            if wl.varlen:
                lens = I.draw_lengths(np.random.default_rng(wl.seed), wl.B, wl.len_lo, wl.len_hi)
                cu_h = np.zeros(len(lens) + 1, dtype=np.int32)
                cu_h[1:] = np.cumsum(lens)
                T, Nw = int(cu_h[-1]), int(lens.max())
                qs, ks = (T, wl.Hq, wl.d), (T, wl.Hkv, wl.d)
                cu = torch.from_numpy(cu_h).to(dev)
                lse_w = torch.empty((wl.Hq, T), dtype=torch.float32, device=dev)
            else:
                lens = np.full(wl.B, wl.N)
                Nw = wl.N
                qs, ks = (wl.B, wl.N, wl.Hq, wl.d), (wl.B, wl.N, wl.Hkv, wl.d)
                cu = None
                lse_w = torch.empty((wl.B, wl.Hq, wl.N), dtype=torch.float32, device=dev)
            qw, kw, vw = rnd(qs, wl.seed * 10 + 1), rnd(ks, wl.seed * 10 + 2), rnd(ks, wl.seed * 10 + 3)
            ow = torch.empty_like(qw)
            fwd = lambda: capi.fa_fwd(qw, kw, vw, ow, lse_w, wl.B, wl.Hq, wl.Hkv, Nw, wl.d, int(wl.causal),
                                      wl.scale, cu, stream)
            ent = {}
            reps_f = 5 if Nw >= 8192 else 20
            ms_f = time_it(fwd, reps_f)
            fl = I.counted_flops(lens, wl.Hq, wl.d, wl.causal)
            ent["fwd_ms"] = round(ms_f, 4)
            ent["fwd_tflops"] = round(fl / (ms_f * 1e-3) / 1e12, 1)
            ent["fwd_frac_of_peak"] = round(fl / (ms_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            # the same forward under other options (same inputs, same launch shape)
            for label, opt in FWD_OPTION_TIMINGS.get(name, ()):
                fx = lambda: capi.fa_fwd_ex(qw, kw, vw, ow, lse_w, wl.B, wl.Hq, wl.Hkv, Nw, wl.d, int(wl.causal),
                                            wl.scale, cu, opt, stream)
                ms_x = time_it(fx, reps_f)
                ent[f"fwd_{label}_ms"] = round(ms_x, 4)
                ent[f"fwd_{label}_vs_default"] = round(ms_x / ms_f, 3)
            if wl.kind == "bwd":
                dow = rnd(qs, wl.seed * 10 + 4)
                dqw, dkw, dvw = torch.empty_like(qw), torch.empty_like(kw), torch.empty_like(vw)
                wsb = capi.fa_bwd_workspace_size(wl.B, wl.Hq, wl.Hkv, Nw, wl.d, int(wl.causal), int(wl.varlen))
                wsw = torch.empty(wsb, dtype=torch.uint8, device=dev)
                bwd = lambda: capi.fa_bwd(qw, kw, vw, ow, lse_w, dow, dqw, dkw, dvw, wl.B, wl.Hq, wl.Hkv, Nw, wl.d,
                                          int(wl.causal), wl.scale, cu, wsw, wsb, stream)
                ms_b = time_it(bwd, 5)
                flb = I.counted_flops(lens, wl.Hq, wl.d, wl.causal, backward=True)
                ent["bwd_ms"] = round(ms_b, 4)
                ent["bwd_tflops"] = round(flb / (ms_b * 1e-3) / 1e12, 1)
                ent["bwd_frac_of_peak"] = round(flb / (ms_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                if name == DQ_AB_WORKLOAD:
                    # dQ: the separate pass (what fa_bwd runs) against the fp32 atomic adds a dQ
                    # accumulated from the dK/dV kernel would need, issued alone
                    dq_pass = lambda: capi.fa_bwd_ex(qw, kw, vw, ow, lse_w, dow, dqw, dkw, dvw, wl.B, wl.Hq, wl.Hkv,
                                                     Nw, wl.d, int(wl.causal), wl.scale, cu, wsw, wsb,
                                                     capi.FA_BWD_DQ, stream)
                    ent["dq_pass_ms"] = round(time_it(dq_pass, 5), 4)
                    acc = torch.zeros((wl.B, Nw, wl.Hq, wl.d), dtype=torch.float32, device=dev)
                    atom = lambda: probe.dq_atomics(acc, wl.B, wl.Hq, Nw, wl.d, int(wl.causal), stream)
                    ent["dq_fused_atomics_only_ms"] = round(time_it(atom, 5), 4)
                    del acc
                del dow, dqw, dkw, dvw, wsw
            workloads[name] = ent
            del qw, kw, vw, ow, lse_w
            torch.cuda.empty_cache()

        # 8-bit Q/K forward: E4M3 codes drawn as N(0, 64^2) rounded by PyTorch's float8_e4m3fn
        # conversion (|x| < 448 at these sizes), descale 1/64 for every (sequence, head)
        for name in ("fp8_fwd_b4_h16_n4096_d128", "fp8_fwd_causal_b2_h16_n16384_d128"):
            wl = I.WORKLOADS[name]
            qs, ks = (wl.B, wl.N, wl.Hq, wl.d), (wl.B, wl.N, wl.Hkv, wl.d)
            q8 = (rnd(qs, wl.seed * 10 + 1).float() * 64).to(torch.float8_e4m3fn).view(torch.uint8)
            k8 = (rnd(ks, wl.seed * 10 + 2).float() * 64).to(torch.float8_e4m3fn).view(torch.uint8)
            vw = rnd(ks, wl.seed * 10 + 3)
            qd = torch.full((wl.B, wl.Hq), 1.0 / 64, dtype=torch.float32, device=dev)
            kd = torch.full((wl.B, wl.Hkv), 1.0 / 64, dtype=torch.float32, device=dev)
            ow = torch.empty(qs, dtype=torch.bfloat16, device=dev)
            lw = torch.empty((wl.B, wl.Hq, wl.N), dtype=torch.float32, device=dev)
            f8 = lambda: capi.fa_fwd_fp8(q8, k8, vw, qd, kd, ow, lw, wl.B, wl.Hq, wl.Hkv, wl.N, wl.d,
                                         int(wl.causal), wl.scale, None, stream)
            ms = time_it(f8, 5 if wl.N >= 8192 else 20)
            fl = I.counted_flops(np.full(wl.B, wl.N), wl.Hq, wl.d, wl.causal)
            # the same codes with one descale per 64-token block (all 1/64)
            nb = (wl.N + 63) // 64
            qdb = torch.full((wl.B, wl.Hq, nb), 1.0 / 64, dtype=torch.float32, device=dev)
            kdb = torch.full((wl.B, wl.Hkv, nb), 1.0 / 64, dtype=torch.float32, device=dev)
            f8b = lambda: capi.fa_fwd_fp8_blockscale(q8, k8, vw, qdb, kdb, ow, lw, wl.B, wl.Hq, wl.Hkv, wl.N, wl.d,
                                                     int(wl.causal), wl.scale, None, None, stream)
            ms_b = time_it(f8b, 5 if wl.N >= 8192 else 20)
            workloads[name] = {"fwd_ms": round(ms, 4), "fwd_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                               "fwd_frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "fwd_frac_of_qk8_pv16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_QK8_PV16_TFLOPS, 4),
                               "fwd_blockscale_ms": round(ms_b, 4),
                               "fwd_blockscale_tflops": round(fl / (ms_b * 1e-3) / 1e12, 1)}
            del q8, k8, vw, qd, kd, ow, lw, qdb, kdb
            torch.cuda.empty_cache()

        # split-KV partial results + merge: 512 queries against 131072 keys
        name = "split_causal_b1_hq32_hkv8_nq512_nk131072_d128"
        wl = I.WORKLOADS[name]
        Bs, Nq, Nk, n = wl.B, wl.N, wl.Nk, wl.n_splits
        qw = rnd((Bs, Nq, wl.Hq, wl.d), wl.seed * 10 + 1)
        kw, vw = rnd((Bs, Nk, wl.Hkv, wl.d), wl.seed * 10 + 2), rnd((Bs, Nk, wl.Hkv, wl.d), wl.seed * 10 + 3)
        opw = torch.empty((n, Bs, Nq, wl.Hq, wl.d), dtype=torch.float32, device=dev)
        lpw = torch.empty((n, Bs, wl.Hq, Nq), dtype=torch.float32, device=dev)
        ow = torch.empty((Bs, Nq, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
        lw = torch.empty((Bs, wl.Hq, Nq), dtype=torch.float32, device=dev)
        split = lambda m: capi.fa_fwd_split(qw, kw, vw, opw, lpw, Bs, wl.Hq, wl.Hkv, Nq, Nk, wl.d, int(wl.causal),
                                            wl.scale, m, stream)
        merge = lambda: capi.fa_merge(opw, lpw, ow, lw, n, Bs, wl.Hq, Nq, wl.d, stream)
        fl = 4.0 * wl.Hq * wl.d * Bs * I.visible_pairs(Nq, Nk, wl.causal)
        ms_1 = time_it(lambda: split(1), 5)          # one chunk: 2 query tiles x 32 heads = 64 workgroups
        ms_s = time_it(lambda: split(n), 5)
        ms_m = time_it(merge, 20)
        rows = Bs * wl.Hq * Nq
        merge_bytes = n * rows * (wl.d + 1) * 4 + rows * (wl.d * 2 + 4)
        workloads[name] = {
            "one_chunk_ms": round(ms_1, 4), "one_chunk_tflops": round(fl / (ms_1 * 1e-3) / 1e12, 1),
            "split_ms": round(ms_s, 4), "split_tflops": round(fl / (ms_s * 1e-3) / 1e12, 1),
            "merge_ms": round(ms_m, 4), "merge_gbs": round(merge_bytes / (ms_m * 1e-3) / 1e9, 1),
            "split_plus_merge_tflops": round(fl / ((ms_s + ms_m) * 1e-3) / 1e12, 1),
            "split_plus_merge_frac_of_peak": round(fl / ((ms_s + ms_m) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        }
        del qw, kw, vw, opw, lpw, ow, lw
        torch.cuda.empty_cache()

    # ---------------- library reference points (child process) ----------------
    reference = None if args.main_only else _library_reference_child()

    # ---------------- CPU oracle baseline (bounded sample) ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
            cores = int(blas[0]["num_threads"]) if blas else os.cpu_count()
        except Exception:
            cores = os.cpu_count()
        # Heads of the same workload, one (batch, head) pair at a time, until
        # about 12 s of oracle work (or --cpu-heads pairs, or all of them).
        f64 = I.bf16_bits_to_f64
        pairs = [(b, hh) for b in range(B) for hh in range(Hq)]
        budget = 12.0
        secs, done = 0.0, 0
        for (b, hh) in pairs:
            if args.cpu_heads and done >= args.cpu_heads:
                break
            if not args.cpu_heads and secs >= budget:
                break
            g = hh // (Hq // Hkv)
            qh = f64(x.q[b:b + 1, :, hh:hh + 1])
            kh, vh = f64(x.k[b:b + 1, :, g:g + 1]), f64(x.v[b:b + 1, :, g:g + 1])
            doh = f64(x.do[b:b + 1, :, hh:hh + 1])
            c0 = time.perf_counter()
            oracle.attention_forward(qh, kh, vh, scale, bool(causal))
            oracle.attention_backward(qh, kh, vh, doh, scale, bool(causal))
            secs += time.perf_counter() - c0
            done += 1
        fl = (I.counted_flops([N], done, d, bool(causal)) +
              I.counted_flops([N], done, d, bool(causal), backward=True))
        cpu = {"value": round(fl / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "seconds": round(secs, 2),
               "sample": f"float64 NumPy oracle, forward + backward of {done} of the {B * Hq} (batch, head) "
                         f"pairs of the same workload (N={N}, d={d}), one pair per call, counted FLOP / oracle "
                         f"wall time"}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"attention forward + backward, B={B}, Hq={Hq}, Hkv={Hkv}, N={N}, d={d}, "
                               f"{'causal' if causal else 'non-causal'} (seeded N(0,1) bf16 inputs)",
                   "global_batch": B, "seq_len": N, "heads_q": Hq, "heads_kv": Hkv, "head_dim": d,
                   "causal": bool(causal), "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
        "workloads": workloads,
        "library_reference": reference,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
