"""Summaries of rocprofv3 output for the attention kernels, as Markdown or key: value text.

    python -m exact_attention_48_amd.profile_summary trace --csv OUT/x_kernel_trace.csv [--skip N]
    python -m exact_attention_48_amd.profile_summary counters --csv OUT/p1_counter_collection.csv \
        --csv OUT/p2_counter_collection.csv
    python -m exact_attention_48_amd.profile_summary traffic --kernel K --workload W \
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv

trace     per-kernel call count, mean / median / min / max duration (us) from a
          ``--kernel-trace`` CSV; ``--skip N`` drops the first N dispatches of every
          kernel (the cold ones) so that the figures describe warm calls, ``--last N``
          keeps only the last N (the calls after a warm-up of any length).
counters  per-kernel means over the profiled dispatches of ``--pmc`` CSVs (several
          passes may be given, one per file), with derived figures:
          cycles = GRBM_GUI_ACTIVE / 8 (it is summed over the 8 XCDs), clock =
          cycles / duration, MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x
          cycles), VALU busy = SQ_ACTIVE_INST_VALU / (256 CUs x cycles) (the
          VALUBusy expression rocprofv3 lists), MFMA TFLOP = 512 x
          SQ_INSTS_VALU_MFMA_MOPS_BF16 (plus 512 x ..._F8), LDS conflict =
          SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE, and issue / wait / issue stall =
          SQ_ACTIVE_INST_ANY, SQ_WAIT_ANY, SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES.
traffic   HBM bytes per launch of one kernel from a FETCH_SIZE and a WRITE_SIZE pass
          (KiB per dispatch), each scaled by what the same counter reads for the
          512 MiB device copy of ``profile_run --part copy``; prints the key: value
          file that bench.py reads, with the kernel's current source hash.
Kernel names are shortened to the function name inside namespace ``fa``; other
kernels (a library's) are kept only when ``--include LABEL=REGEX`` matches their
name, and are then listed under LABEL.
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import statistics
import sys

from .kernel_sources import source_hash

COPY_BYTES = 512 << 20


_INCLUDE = []   # (label, compiled regex) for kernels outside namespace fa


def _short(name: str):
    m = re.search(r"fa::(\w+)(<[^()]*>)?", name)
    if not m:
        for label, rx in _INCLUDE:
            if rx.search(name):
                return label
        return None
    return m.group(1) + (m.group(2) or "")


def _base(short: str) -> str:
    return short.split("<", 1)[0]


def trace(args):
    durs = collections.OrderedDict()
    with open(args.csv) as fh:
        for r in csv.DictReader(fh):
            k = _short(r["Kernel_Name"])
            if k is None:
                continue
            durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | calls | mean (us) | median (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|")
    for k, v in durs.items():
        w = v[args.skip:] if len(v) > args.skip else v
        if args.last:
            w = w[-args.last:]
        print(f"| `{k}` | {len(w)} | {statistics.mean(w):.1f} | {statistics.median(w):.1f} | {min(w):.1f} | "
              f"{max(w):.1f} |")
    if args.skip:
        print(f"\n(first {args.skip} dispatch(es) of each kernel dropped)")
    if args.last:
        print(f"\n(the last {args.last} dispatch(es) of each kernel)")


def _counter_means(paths):
    """kernel -> counter -> mean over dispatches (each dispatch's value summed over its
    dimension rows), plus kernel -> mean duration (ns)."""
    vals = collections.OrderedDict()
    durs = collections.defaultdict(dict)
    for p in paths:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        with open(p) as fh:
            for r in csv.DictReader(fh):
                k = _short(r["Kernel_Name"])
                if k is None:
                    continue
                did = int(r["Dispatch_Id"])
                per[(k, r["Counter_Name"])][did] += float(r["Counter_Value"])
                durs[k][(p, did)] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for (k, c), d in per.items():
            vals.setdefault(k, {})[c] = sum(d.values()) / len(d)
    return vals, {k: sum(v.values()) / len(v) for k, v in durs.items()}


def counters(args):
    vals, durs = _counter_means(args.csv)
    cols = ["us", "GHz", "MFMA busy", "VALU busy", "MFMA TFLOP", "MFMA TFLOP/s", "VALU instr", "of which trans",
            "MFMA instr", "LDS instr", "SALU instr", "LDS conflict", "issue", "s_waitcnt", "issue stall"]
    print("| kernel | " + " | ".join(cols) + " |")
    print("|---|" + "---|" * len(cols))
    for k, c in vals.items():
        ns = durs[k]
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        row = [f"{ns / 1e3:.1f}", f"{cyc / ns:.2f}" if cyc else "-"]

        def pct(num, den):
            return f"{100.0 * num / den:.1f} %" if den else "-"
        row.append(pct(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), 1024 * cyc) if "SQ_VALU_MFMA_BUSY_CYCLES" in c else "-")
        row.append(pct(c["SQ_ACTIVE_INST_VALU"], 256 * cyc) if "SQ_ACTIVE_INST_VALU" in c and cyc else "-")
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        has_mops = "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c
        row.append(f"{512 * mops / 1e12:.3f}" if has_mops else "-")
        row.append(f"{512 * mops / (ns * 1e-9) / 1e12:.0f}" if has_mops else "-")
        for n in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            row.append(f"{c[n]:.3g}" if n in c else "-")
        row.append(pct(c["SQ_LDS_BANK_CONFLICT"], c["SQ_LDS_IDX_ACTIVE"]) if "SQ_LDS_BANK_CONFLICT" in c
                   and "SQ_LDS_IDX_ACTIVE" in c else "-")
        for n in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"):
            row.append(pct(c[n], c["SQ_WAVE_CYCLES"]) if n in c and "SQ_WAVE_CYCLES" in c else "-")
        print(f"| `{k}` | " + " | ".join(row) + " |")


def _one_counter(path, counter, kernel=None):
    vals, _ = _counter_means([path])
    if kernel is None:   # the copy run: the largest value of any kernel (the copy itself)
        with open(path) as fh:
            per = collections.defaultdict(float)
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        return max(per.values())
    for k, c in vals.items():
        if _base(k) == kernel and counter in c:
            return c[counter]
    raise SystemExit(f"{counter} of {kernel} not found in {path}")


def traffic(args):
    f = _one_counter(args.fetch, "FETCH_SIZE", args.kernel)
    w = _one_counter(args.write, "WRITE_SIZE", args.kernel)
    cf = _one_counter(args.copy_fetch, "FETCH_SIZE")
    cw = _one_counter(args.copy_write, "WRITE_SIZE")
    fs, ws = (COPY_BYTES / 1024) / cf, (COPY_BYTES / 1024) / cw
    print(f"kernel: {args.kernel}")
    print(f"workload: {args.workload}")
    print(f"fetch_size_kib: {f:.0f}")
    print(f"write_size_kib: {w:.0f}")
    print(f"copy_fetch_size_kib_for_512MiB: {cf:.0f}")
    print(f"copy_write_size_kib_for_512MiB: {cw:.0f}")
    print(f"fetch_scale: {fs:.4f}")
    print(f"write_scale: {ws:.4f}")
    print(f"hbm_bytes_per_launch: {(f * fs + w * ws) * 1024:.0f}")
    print(f"source_hash: {source_hash(args.kernel)}")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", required=True)
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--last", type=int, default=0, help="keep only the last N dispatches of each kernel")
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True)
    r = sub.add_parser("traffic")
    for n in ("kernel", "workload", "fetch", "write", "copy-fetch", "copy-write"):
        r.add_argument("--" + n, required=True)
    for p in (t, c):
        p.add_argument("--include", action="append", default=[], metavar="LABEL=REGEX")
    args = ap.parse_args(argv)
    _INCLUDE.clear()
    for spec in getattr(args, "include", []):
        label, _, rx = spec.partition("=")
        if not label or not rx:
            raise SystemExit(f"--include wants LABEL=REGEX, got {spec!r}")
        _INCLUDE.append((label, re.compile(rx)))
    {"trace": trace, "counters": counters, "traffic": traffic}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
