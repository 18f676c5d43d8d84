"""CPU checks of bench.py's profile summarisers: rocprofv3 CSV output and bench
lines in, the profiles/ tables and the traffic record out.  Inputs are tiny
synthetic files whose figures are chosen so the expected table entries are
known exactly; the summaries are written to a temporary directory."""
import csv
import json
import os

import pytest

import bench

KBWD = "void flce::k_bwd<flce::BF16>(flce::BwdArgs, flce::BwdArgs, int, int, int, int)"
COPY = "void at::native::copyBuffer(long)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


@pytest.fixture
def out(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    monkeypatch.setattr(bench, "TRAFFIC", str(prof / "traffic.json"))
    return tmp_path


def test_mfma_summary_normalises_by_xcds_and_simds(out):
    ns = 1_000_000                       # one 1 ms dispatch
    clock = 1.7e9                        # cycles per second of one XCD
    gui = 8 * clock * ns * 1e-9          # GRBM_GUI_ACTIVE comes summed over 8 XCDs
    busy = 0.75 * (gui / 8) * 1024       # matrix cores busy 75 % of the cycles
    mops = 1.3e15 * ns * 1e-9 / 512      # 1.3 PFLOP/s of bf16 MFMA work
    base = dict(Dispatch_Id=7, Kernel_Name=KBWD, Start_Timestamp=0, End_Timestamp=ns)
    _write(str(out / "run" / "prof_mfma" / "a_counter_collection.csv"),
           [dict(base, Counter_Name=c, Counter_Value=v)
            for c, v in (("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                         ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops))])
    _write(str(out / "run" / "prof_mfma" / "a_kernel_trace.csv"),
           [dict(Dispatch_Id=7, Start_Timestamp=0, End_Timestamp=ns)])
    bench.summarize_mfma(str(out / "run"))
    md = open(out / "profiles" / "flce_qwen2_7b_head_mfma.md").read()
    row = [l for l in md.splitlines() if l.startswith("| k_bwd<BF16> |")]
    assert len(row) == 1, md
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # kernel, dispatches, avg us, busy, clock, TFLOP/launch, TFLOP/s, % of 2.5 PF, % at clock
    assert cells[1:5] == ["1", "1000.0", "75.0 %", "1.70"]
    assert cells[6] == "1300"
    assert cells[7] == "52.0"
    assert float(cells[8]) == pytest.approx(100 * 1.3 / (2.5 * 1.7 / 2.4), abs=0.06)


def test_traffic_summary_scales_by_the_copy_calibration(out):
    run = out / "run"
    _write(str(run / "prof_trace" / "a_kernel_stats.csv"),
           [dict(Name=KBWD, Calls=2, TotalDurationNs=3e6, AverageNs=1.5e6, Percentage=90.0)])
    gib_kib = float(1 << 20)
    for sub, counter, calib, per in (("prof_fetch", "FETCH_SIZE", gib_kib / 2, 1000.0),
                                     ("prof_write", "WRITE_SIZE", gib_kib, 250.0)):
        _write(str(run / sub / "a_counter_collection.csv"),
               [dict(Kernel_Name=COPY, Counter_Name=counter, Counter_Value=calib,
                     Grid_Size=131072),
                dict(Kernel_Name=KBWD, Counter_Name=counter, Counter_Value=per, Grid_Size=512),
                dict(Kernel_Name=KBWD, Counter_Name=counter, Counter_Value=per, Grid_Size=512)])
    bench.summarize(str(run), ("cmd",))
    t = json.load(open(out / "profiles" / "traffic.json"))
    assert t["source_hash"] == bench.source_hash()
    assert t["calibration"] == {"fetch": 2.0, "write": 1.0}
    # fetch KiB per dispatch x 1024 x 2 (the copy reads half of its GiB) + write KiB x 1024
    assert t["bytes_per_launch"]["k_bwd"] == pytest.approx(1000.0 * 1024 * 2 + 250.0 * 1024)
    md = open(out / "profiles" / "flce_qwen2_7b_head_kernels.md").read()
    assert "| k_bwd<BF16> | 2 | 3.000 | 1500.0 | 90.00 |" in md


def test_workload_table_has_one_row_per_bench_line(out):
    run = out / "run"
    run.mkdir()
    line = {"config": {"workload": "qwen2_7b_head: N=8192"}, "ms_per_step": 22.5,
            "value": 364088.9, "mfma_frac_model": 0.4761, "peak_extra_bytes": 1.86e9,
            "dtype": "bf16",
            "chunked_mode": {"ms_per_step": 18.0, "mfma_frac_model": 0.595},
            "torch_eager": {"ms_per_step": 34.0, "peak_extra_bytes": 1.49e10},
            "vendor_gemm": {"ms": 5.05}, "cpu_baseline": {"value": 390.2}}
    tiny = {"config": {"workload": "tiny_f32: N=128"}, "ms_per_step": 0.05, "value": 2.56e6,
            "mfma_frac_model": 0.0161, "peak_extra_bytes": 3.0e6, "dtype": "f32",
            "chunked_mode": {"ms_per_step": 0.04, "mfma_frac_model": 0.0201},
            "cpu_baseline": {"value": 5000.0}}
    with open(run / "bench_qwen2_7b_head.json", "w") as f:
        f.write("[bench] progress line\n" + json.dumps(line) + "\n")
    with open(run / "bench_tiny_f32.json", "w") as f:
        f.write(json.dumps(tiny) + "\n")
    bench.summarize_workloads(str(run))
    md = open(out / "profiles" / "flce_workloads_bench.md").read()
    rows = [l for l in md.splitlines() if l.startswith("| qwen2_7b_head") or
            l.startswith("| tiny_f32")]
    # one row per bench line, each against its own dtype's dense peak
    assert rows == ["| tiny_f32: N=128 | 0.05 | 2.56e+06 | 157.3 | 1.6 | 0.00 | 0.04 | 2.0 | "
                    "nan | nan | nan | 5000 |",
                    "| qwen2_7b_head: N=8192 | 22.50 | 3.64e+05 | 2500 | 47.6 | 1.86 | 18.00 | "
                    "59.5 | 34.00 | 14.9 | 5.05 | 390 |"]


def test_ceiling_summary_keeps_the_probe_table(out):
    table = ["| operands | TFLOP/s | % of 2500 TFLOP/s | clock at 100 % busy (GHz) |",
             "|---|---|---|---|",
             "| constant operands (1.0) | 2434 | 97.4 | 2.34 |",
             "| random sign and mantissa, one exponent (2^-7) | 1900 | 76.0 | 1.82 |"]
    (out / "mfma_ceiling.txt").write_text("\n".join(["probe noise"] + table) + "\n")
    md = open(bench.summarize_ceiling(str(out))).read()
    for row in table:
        assert row in md
    assert "mfma_ceiling > $R/gpurun_out/mfma_ceiling.txt" in md
    (out / "mfma_ceiling.txt").write_text("no table\n")
    with pytest.raises(SystemExit):
        bench.summarize_ceiling(str(out))
