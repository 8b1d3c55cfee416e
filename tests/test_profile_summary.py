"""The rocprofv3 summariser (host logic): synthetic CSVs with known answers."""
import csv
import io
import contextlib

import pytest

from exact_attention_48_amd import kernel_sources, profile_summary as PS

TRACE_COLS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
FWD = "void fa::fa_fwd_pp_kernel<false, false, 0>(fa::FwdParams)"
DKDV = "void fa::bwd_dkdv_kernel<128, false, false>(fa::BwdParams)"


def _write(path, cols, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _run(argv):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        PS.main(argv)
    return buf.getvalue()


def test_trace_drops_cold_calls(tmp_path):
    rows = []
    t = 0
    for us in (900, 100, 110, 120, 130):          # one cold call, then warm ones
        rows.append({"Kernel_Name": FWD, "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
        t += 10 ** 7
    rows.append({"Kernel_Name": "void other_kernel()", "Start_Timestamp": 0, "End_Timestamp": 5})
    p = tmp_path / "k_kernel_trace.csv"
    _write(p, TRACE_COLS, rows)
    out = _run(["trace", "--csv", str(p), "--skip", "1"])
    line = [l for l in out.splitlines() if "fa_fwd_pp_kernel" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[0] == "`fa_fwd_pp_kernel<false, false, 0>`"
    assert cells[1:] == ["4", "115.0", "115.0", "100.0", "130.0"]
    assert "other_kernel" not in out
    all_calls = _run(["trace", "--csv", str(p)])
    assert "| 5 | 272.0 |" in all_calls


def test_counters_derived_figures(tmp_path):
    # two dispatches of one kernel, each counter split over two dimension rows (summed per dispatch)
    dur_ns = 500_000
    cyc = 1_000_000                                   # cycles per XCD -> 2.0 GHz
    vals = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * cyc,
            "SQ_ACTIVE_INST_VALU": 0.25 * 256 * cyc, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e9,
            "SQ_INSTS_VALU": 1e8, "SQ_INSTS_VALU_TRANS_F32": 2e7, "SQ_LDS_BANK_CONFLICT": 10.0,
            "SQ_LDS_IDX_ACTIVE": 1000.0, "SQ_WAVE_CYCLES": 4e8, "SQ_ACTIVE_INST_ANY": 2e8,
            "SQ_WAIT_ANY": 1e8, "SQ_WAIT_INST_ANY": 1e8}
    rows = []
    for did in (1, 2):
        for name, v in vals.items():
            for half in (0, 1):
                rows.append({"Dispatch_Id": did, "Kernel_Name": DKDV, "Counter_Name": name, "Counter_Value": v / 2,
                             "Start_Timestamp": 0, "End_Timestamp": dur_ns})
    p = tmp_path / "p_counter_collection.csv"
    _write(p, PMC_COLS, rows)
    out = _run(["counters", "--csv", str(p)])
    header = [c.strip() for c in out.splitlines()[0].strip("|").split("|")]
    line = [l for l in out.splitlines() if "bwd_dkdv_kernel" in l][0]
    got = dict(zip(header, [c.strip() for c in line.strip("|").split("|")]))
    assert got["us"] == "500.0" and got["GHz"] == "2.00"
    assert got["MFMA busy"] == "50.0 %" and got["VALU busy"] == "25.0 %"
    assert got["MFMA TFLOP"] == "1.024"                # 512 x 2e9
    assert got["MFMA TFLOP/s"] == "2048"               # 1.024e12 / 500 us
    assert got["of which trans"] == "2e+07" and got["LDS conflict"] == "1.0 %"
    assert got["issue"] == "50.0 %" and got["s_waitcnt"] == "25.0 %" and got["issue stall"] == "25.0 %"


def test_traffic_scales_by_the_copy(tmp_path):
    def pmc(path, name, counter, kib):
        _write(path, PMC_COLS, [{"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib,
                                 "Start_Timestamp": 0, "End_Timestamp": 1} for d in (1, 2)])
    copy = "void at::native::elementwise_kernel<copy>()"
    pmc(tmp_path / "f.csv", DKDV, "FETCH_SIZE", 1000.0)
    pmc(tmp_path / "w.csv", DKDV, "WRITE_SIZE", 300.0)
    pmc(tmp_path / "cf.csv", copy, "FETCH_SIZE", (512 << 10) / 2)   # the copy reads FETCH_SIZE at half
    pmc(tmp_path / "cw.csv", copy, "WRITE_SIZE", 512 << 10)
    out = _run(["traffic", "--kernel", "bwd_dkdv_kernel", "--workload", "w", "--fetch", str(tmp_path / "f.csv"),
                "--write", str(tmp_path / "w.csv"), "--copy-fetch", str(tmp_path / "cf.csv"),
                "--copy-write", str(tmp_path / "cw.csv")])
    kv = dict(l.split(": ", 1) for l in out.splitlines())
    assert kv["fetch_scale"] == "2.0000" and kv["write_scale"] == "1.0000"
    assert int(kv["hbm_bytes_per_launch"]) == (2 * 1000 + 300) * 1024
    assert kv["source_hash"] == kernel_sources.source_hash("bwd_dkdv_kernel")


@pytest.mark.parametrize("kernel", sorted(kernel_sources.KERNEL_SOURCES))
def test_source_hash_is_stable(kernel):
    h = kernel_sources.source_hash(kernel)
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == kernel_sources.source_hash(kernel)


def test_library_kernels_only_when_included(tmp_path):
    lib = "Cijk_Alik_Bljk_BBS_BH_MT256x256x64_MI16x16x1"
    rows = [{"Kernel_Name": lib, "Start_Timestamp": 0, "End_Timestamp": 800_000},
            {"Kernel_Name": FWD, "Start_Timestamp": 0, "End_Timestamp": 400_000}]
    p = tmp_path / "g_kernel_trace.csv"
    _write(p, TRACE_COLS, rows)
    assert "Cijk" not in _run(["trace", "--csv", str(p)])
    out = _run(["trace", "--csv", str(p), "--include", "gemm_bf16=^Cijk_"])
    line = [l for l in out.splitlines() if l.startswith("| `gemm_bf16`")][0]
    assert "| 1 | 800.0 |" in line
    assert "fa_fwd_pp_kernel" in out
    with pytest.raises(SystemExit):
        _run(["trace", "--csv", str(p), "--include", "no-regex"])


def test_trace_last_keeps_the_final_calls(tmp_path):
    rows = []
    t = 0
    for us in (900, 800, 700, 100, 110, 120):
        rows.append({"Kernel_Name": FWD, "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
        t += 10 ** 7
    p = tmp_path / "w_kernel_trace.csv"
    _write(p, TRACE_COLS, rows)
    line = [l for l in _run(["trace", "--csv", str(p), "--last", "3"]).splitlines() if "fa_fwd_pp_kernel" in l][0]
    assert [c.strip() for c in line.strip("|").split("|")][1:] == ["3", "110.0", "110.0", "100.0", "120.0"]


def test_code_only_ignores_comments_not_code():
    a = 'int f(int x) { // add one\n  return x + 1; /* done */ }\nconst char* s = "a // b";\n'
    b = 'int f(int x) {\n\n  return x + 1;   }\n// a comment\nconst char* s = "a // b";'
    assert kernel_sources.code_only(a) == kernel_sources.code_only(b)
    assert "a // b" in kernel_sources.code_only(a)              # inside a string: code
    c = 'int f(int x) { return x + 2; }\nconst char* s = "a // b";'
    assert kernel_sources.code_only(a) != kernel_sources.code_only(c)
    assert kernel_sources.code_only("x = '\\'';  // q") == "x = '\\'';"
