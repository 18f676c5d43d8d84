#!/usr/bin/env python3
"""Fused linear cross-entropy forward + backward on one MI355X.

One step = flce_forward + flce_backward (every kernel of the path) over one
batch of synthetic input already resident in HBM.  The default workload is the
Qwen2-7B-like LM head: B=1, T=8192 (N=8192 rows), H=3584, V=152064, bf16,
Zipf(1.1) labels, first 20% of the sequence masked, next-token shift, mean.

Prints ONE JSON line with the throughput (tokens/s over all N rows), the
fraction of the bf16 dense MFMA peak on the 6NHV model-FLOP basis, the peak
extra device memory, a roofline entry for the dominant kernel (its average
launch duration measured with HIP events on its own stream inside the timed
region) and the float64 oracle timed on the host cores on a bounded row sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
F32_PEAK = 157.3e12       # MI355X dense fp32 MFMA, FLOP/s
HBM_PEAK = 8.0e12         # MI355X HBM3E, B/s
KERNELS = ("k_fwd_lse", "k_bwd")
# MFMA contractions per step of each kernel, in units of 2 n H V flops: the
# forward logits; the backward's recomputed logits, dX and dW
GEMMS_PER_STEP = {"k_fwd_lse": 1, "k_bwd": 3}
KERNEL_SOURCES = ("lm_head_linear_flce_amd/csrc/flce_tile.h",
                  "lm_head_linear_flce_amd/csrc/flce_kernels.h",
                  "lm_head_linear_flce_amd/csrc/flce_api.hip")
PROFILES = os.path.join(ROOT, "profiles")
# the rocprofv3 runs the committed summaries come from ($R = repository root,
# run from /tmp with TMPDIR=/tmp)
PROFILE_COMMANDS = (
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_trace -o flce "
    "-- python $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-chunked --no-vendor-gemm --no-torch-reference",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof_fetch -o flce "
    "-- python $R/bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-chunked --no-vendor-gemm --no-torch-reference "
    "--copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof_write -o flce "
    "-- python $R/bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-chunked --no-vendor-gemm --no-torch-reference "
    "--copy-calibration",
    "python $R/bench.py --summarize $R/gpurun_out",
)
# the chunked mode's own kernel trace (profiles/flce_qwen2_7b_head_chunked_kernels.md)
CHUNKED_PROFILE_COMMANDS = (
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_chunk -o flce "
    "-- python $R/bench.py --steps 3 --warmup 1 --chunked-only",
    "python $R/bench.py --summarize-chunked $R/gpurun_out",
)
# matrix-core busy cycles, bf16 MFMA work and the shader clock per kernel
# (profiles/flce_qwen2_7b_head_mfma.md); each counter run holds 3 SQ and 1 GRBM
# counters, with the kernel trace for the durations
MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
MFMA_PROFILE_COMMANDS = (
    f"rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv "
    "-d $R/gpurun_out/prof_mfma -o flce -- python $R/bench.py --steps 1 --warmup 0 "
    "--no-cpu-baseline --no-chunked --no-vendor-gemm --no-torch-reference",
    f"rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv "
    "-d $R/gpurun_out/prof_mfma_chunk -o flce -- python $R/bench.py --steps 1 --warmup 0 "
    "--chunked-only",
    *(f"rocprofv3 --pmc {c} --kernel-trace --output-format csv -d $R/gpurun_out/stall{i + 1} "
      "-o flce -- python $R/bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-chunked --no-vendor-gemm --no-torch-reference"
      for i, c in enumerate((
          "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_INSTS_VMEM_RD "
          "SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL GRBM_GUI_ACTIVE",
          "SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_LDS_BANK_CONFLICT "
          "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE",
          "SQ_WAVE_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_SALU SQ_ACTIVE_INST_SCA "
          "SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL GRBM_GUI_ACTIVE"))),
    f"rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv "
    "-d $R/gpurun_out/prof_mfma_vendor -o flce -- python $R/bench.py --steps 2 --warmup 1 "
    "--vendor-gemm-only",
    "python $R/bench.py --summarize-mfma $R/gpurun_out",
)
# the matrix cores' sustained rate with no memory traffic, by operand data
# (profiles/mfma_ceiling.md): context for the roofline's published peak
CEILING_COMMANDS = (
    "$R/lm_head_linear_flce_amd/mfma_ceiling > $R/gpurun_out/mfma_ceiling.txt",
    "python $R/bench.py --summarize-ceiling $R/gpurun_out",
)
# every bf16 workload through the bench (profiles/flce_workloads_bench.md)
BENCH_WORKLOADS = ("tiny_f32", "qwen2_7b_head", "qwen3_sft_batch", "long_context", "ragged_vocab")
WORKLOAD_BENCH_COMMANDS = tuple(
    f"python $R/bench.py --workload {name} --steps 5 --warmup 2 > $R/gpurun_out/bench_{name}.json"
    for name in BENCH_WORKLOADS) + ("python $R/bench.py --summarize-workloads $R/gpurun_out",)
SIMDS = 256 * 4           # MI355X: 256 compute units x 4 SIMDs
XCDS = 8                  # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
TRAFFIC = os.path.join(PROFILES, "traffic_qwen2_7b_head.json")
METRIC = "fused linear-CE fwd+bwd tokens/sec and % bf16 MFMA peak; peak extra HBM bytes"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen2_7b_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-mode measurement")
    ap.add_argument("--chunk-rows", type=int, default=0,
                    help="rows per chunk of the chunked mode (0 = as many as a 2 GiB slab holds)")
    ap.add_argument("--chunked-only", action="store_true",
                    help="measure only the chunked mode and print its figures (for "
                         "CHUNKED_PROFILE_COMMANDS)")
    ap.add_argument("--summarize-chunked", metavar="DIR",
                    help="summarise DIR/prof_chunk of CHUNKED_PROFILE_COMMANDS into profiles/")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="summarise DIR/prof_mfma and DIR/prof_mfma_chunk of "
                         "MFMA_PROFILE_COMMANDS into profiles/")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip timing hipBLASLt on the forward's logits GEMM")
    ap.add_argument("--vendor-gemm-only", action="store_true",
                    help="time only hipBLASLt on the forward's logits GEMM (for the "
                         "counter runs)")
    ap.add_argument("--no-torch-reference", action="store_true",
                    help="skip timing the same loss in PyTorch eager")
    ap.add_argument("--summarize-workloads", metavar="DIR",
                    help="summarise DIR/bench_<workload>.json of WORKLOAD_BENCH_COMMANDS into "
                         "profiles/")
    ap.add_argument("--summarize-ceiling", metavar="DIR",
                    help="wrap DIR/mfma_ceiling.txt of CEILING_COMMANDS into profiles/")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--summarize", metavar="DIR",
                    help="summarise the rocprofv3 output of PROFILE_COMMANDS under DIR "
                         "(DIR/prof_trace, DIR/prof_fetch, DIR/prof_write) into "
                         "profiles/ and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy first (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none for this workload or the kernels changed since."""
    if workload != "qwen2_7b_head" or not os.path.exists(TRAFFIC):
        return None
    with open(TRAFFIC) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t["bytes_per_launch"].get(kernel)


def oracle_baseline(w, rows_wanted):
    """The float64 oracle on a bounded sample of valid rows (full per-row work:
    logits rows, softmax, dX rows and their dW contribution), extrapolated to
    the workload's valid rows."""
    import numpy as np

    import oracle
    y, valid = oracle.targets(w.labels, w.shift, w.ignore_index)
    vrows = np.flatnonzero(valid)
    n = len(vrows)
    r = min(rows_wanted, n)
    pick = vrows[np.linspace(0, n - 1, r).astype(np.int64)]
    Xs = w.X[pick]
    ys = y[pick].reshape(1, -1)
    t0 = time.perf_counter()
    oracle.flce(Xs, w.W, ys, ignore_index=w.ignore_index, reduction=w.reduction,
                shift=False, mode="global")
    t = time.perf_counter() - t0
    t_full = t * n / r
    cores = len(os.sched_getaffinity(0))
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            cores = min(cores, int(os.environ[var]))
            break
    return {
        "value": w.N / t_full, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": f"{r} of {n} valid rows of the {w.N}x{w.H}x{w.V} workload, forward + "
                  f"backward in float64 numpy ({t:.1f} s), time scaled by {n}/{r}",
    }


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name):
    import re
    name = re.sub(r"\(.*", "", name).replace("void ", "")
    return name.replace("flce::", "")


def summarize(prof_dir, command, trace="prof_trace", out="flce_qwen2_7b_head_kernels.md",
              title="Kernel time and HBM traffic: Qwen2-7B-like LM head (forward + "
                    "backward)"):
    """Kernel-trace statistics and calibrated HBM traffic -> profiles/."""
    import csv
    import glob
    stats = glob.glob(os.path.join(prof_dir, trace, "**", "*kernel_stats.csv"),
                      recursive=True)
    pmcs = [] if trace != "prof_trace" else [p for sub in ("prof_fetch", "prof_write")
                                             for p in glob.glob(os.path.join(
                                                 prof_dir, sub, "**", "*counter_collection.csv"),
                                                 recursive=True)]
    lines = [f"# {title}, N=8192 H=3584 V=152064 bf16", "",
             f"kernel source hash: `{source_hash()}`", "",
             "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root):", "",
             "```", *command, "```", ""]
    rows = []
    for path in stats:
        for r in csv.DictReader(open(path)):
            rows.append((_short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["Percentage"])))
    rows.sort(key=lambda x: -x[2])
    lines += ["## rocprofv3 --kernel-trace --stats", "",
              "| kernel | calls | total ms | avg us | % |", "|---|---|---|---|---|"]
    for n, c, tot, avg, pct in rows:
        if pct < 0.01:
            continue
        lines.append(f"| {n} | {c} | {tot / 1e6:.3f} | {avg / 1e3:.1f} | {pct:.2f} |")
    # counters: per kernel, per dispatch averages; the 1 GiB copy calibrates
    per = {}
    calib = {}
    for path in pmcs:
        for r in csv.DictReader(open(path)):
            n = _short(r["Kernel_Name"])
            cn = r["Counter_Name"]
            v = float(r["Counter_Value"])
            if "copyBuffer" in n and int(r["Grid_Size"]) == 131072:
                calib[cn] = v
                continue
            d = per.setdefault(n, {}).setdefault(cn, [0.0, 0])
            d[0] += v
            d[1] += 1
    gib_kib = float(1 << 20)
    f_fetch = gib_kib / calib["FETCH_SIZE"] if calib.get("FETCH_SIZE") else None
    f_write = gib_kib / calib["WRITE_SIZE"] if calib.get("WRITE_SIZE") else None
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = "
              f"{calib.get('FETCH_SIZE', float('nan')):.0f} KiB and WRITE_SIZE = "
              f"{calib.get('WRITE_SIZE', float('nan')):.0f} KiB; scale factors "
              f"{f_fetch} and {f_write}.", "",
              "| kernel | dispatches | fetch MB / launch | write MB / launch | traffic MB / launch |",
              "|---|---|---|---|---|"]
    traffic = {}
    for n, d in sorted(per.items()):
        if not any(k in n for k in KERNELS) or "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        fe = d["FETCH_SIZE"][0] / d["FETCH_SIZE"][1] * 1024 * (f_fetch or 1.0)
        wr = d["WRITE_SIZE"][0] / d["WRITE_SIZE"][1] * 1024 * (f_write or 1.0)
        key = n.split("<")[0]
        traffic[key] = fe + wr
        lines.append(f"| {n} | {d['FETCH_SIZE'][1]} | {fe / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(fe + wr) / 1e6:.1f} |")
    os.makedirs(PROFILES, exist_ok=True)
    md = os.path.join(PROFILES, out)
    if not pmcs:
        os.makedirs(PROFILES, exist_ok=True)
        with open(md, "w") as f:
            f.write("\n".join(lines[:lines.index("## HBM traffic (rocprofv3 --pmc FETCH_SIZE, "
                                                   "then --pmc WRITE_SIZE)")]) + "\n")
        print(md)
        return
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(TRAFFIC, "w") as f:
        json.dump({"source_hash": source_hash(), "bytes_per_launch": traffic,
                   "calibration": {"fetch": f_fetch, "write": f_write}}, f, indent=1)
    print(md)


def summarize_mfma(prof_dir):
    """Per kernel and dispatch: matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES
    over GRBM_GUI_ACTIVE x SIMDs), bf16 MFMA flops counted by the hardware
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), the shader clock (GRBM_GUI_ACTIVE over
    the dispatch's duration) and the achieved rate -> profiles/."""
    import csv
    import glob
    out = ["# MFMA utilisation and shader clock: Qwen2-7B-like LM head, N=8192 H=3584 "
           "V=152064 bf16", "", f"kernel source hash: `{source_hash()}`", "",
           "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root):", "",
           "```", *MFMA_PROFILE_COMMANDS, "```", "",
           "Per dispatch: GRBM_GUI_ACTIVE is reported summed over the 8 XCDs, so one "
           "XCD's busy cycles are a = GRBM_GUI_ACTIVE / 8 (the memory-bound bf16 copy "
           "kernel's row reads 2.40 GHz, the top clock); MFMA busy = "
           "SQ_VALU_MFMA_BUSY_CYCLES / (a x 1024 SIMDs); MFMA flop = "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the padded tiles' work: rows rounded up "
           "to 256); clock = a / duration; rate = MFMA flop / duration; the peak at the "
           "measured clock is 2.5 PFLOP/s x clock / 2.4 GHz. Dispatches under 50 us are "
           "left out.", ""]
    for sub, title in (("prof_mfma", "recompute path (flce_forward + flce_backward)"),
                       ("prof_mfma_chunk", "chunked mode (flce_chunked)"),
                       ("prof_mfma_vendor", "reference point: hipBLASLt on the forward's "
                                            "logits GEMM alone (torch.matmul, [n, V] "
                                            "logits materialised)")):
        cc = glob.glob(os.path.join(prof_dir, sub, "**", "*counter_collection.csv"),
                       recursive=True)
        kt = glob.glob(os.path.join(prof_dir, sub, "**", "*kernel_trace.csv"), recursive=True)
        if not cc or not kt:
            continue
        dur = {}
        for path in kt:
            for r in csv.DictReader(open(path)):
                dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        per = {}
        for path in cc:
            for r in csv.DictReader(open(path)):
                d = per.setdefault(r["Dispatch_Id"], {"name": _short(r["Kernel_Name"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        agg = {}
        for did, d in per.items():
            ns = dur.get(did)
            if not ns or ns < 50_000 or "GRBM_GUI_ACTIVE" not in d:
                continue
            a = agg.setdefault(d["name"], [])
            a.append((ns, d["GRBM_GUI_ACTIVE"] / XCDS, d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0),
                      d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512))
        out += [f"## {title}", "",
                "| kernel | dispatches | avg us | MFMA busy | clock GHz | MFMA TFLOP/launch "
                "| TFLOP/s | % of 2.5 PF | % of peak at measured clock |",
                "|---|---|---|---|---|---|---|---|---|"]
        for name, a in sorted(agg.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
            ns = sum(x[0] for x in a) / len(a)
            gui = sum(x[1] for x in a) / len(a)
            busy = sum(x[2] for x in a) / len(a) / (gui * SIMDS)
            fl = sum(x[3] for x in a) / len(a)
            clk = gui / ns
            rate = fl / (ns * 1e-9)
            out.append(f"| {name} | {len(a)} | {ns / 1e3:.1f} | {100 * busy:.1f} % | {clk:.2f} | "
                       f"{fl / 1e12:.3f} | {rate / 1e12:.0f} | {100 * rate / BF16_PEAK:.1f} | "
                       f"{100 * rate / (BF16_PEAK * clk / 2.4):.1f} |")
        out.append("")
    # where the waves' time goes (the stall runs): SQ_WAVE_CYCLES, SQ_WAIT_* and
    # SQ_ACTIVE_INST_* all count wave-cycles in the same units, so their ratios are
    # fractions of the waves' lifetime
    stall = {}
    for i in (1, 2, 3):
        for path in glob.glob(os.path.join(prof_dir, f"stall{i}", "**", "*counter_collection.csv"),
                              recursive=True):
            per = {}
            for r in csv.DictReader(open(path)):
                name = _short(r["Kernel_Name"])
                if not any(k in name for k in KERNELS):
                    continue
                d = per.setdefault(r["Dispatch_Id"], {"name": name})
                d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            for d in per.values():
                if d["ns"] < 50_000 or not d.get("SQ_WAVE_CYCLES"):
                    continue
                acc = stall.setdefault(d["name"], {})
                for c, v in d.items():
                    if c.startswith("SQ_"):
                        acc.setdefault(c, []).append(v / d["SQ_WAVE_CYCLES"] if c != "SQ_WAVE_CYCLES"
                                                     else v)
    if stall:
        rows = (("SQ_WAIT_ANY", "waiting on s_waitcnt / barrier"),
                ("SQ_WAIT_INST_ANY", "waiting to issue (includes the MFMA pipe's back-pressure)"),
                ("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction"),
                ("SQ_ACTIVE_INST_LDS", "LDS instructions active"),
                ("SQ_ACTIVE_INST_VALU", "VALU instructions active (the counter's issue-side count)"),
                ("SQ_ACTIVE_INST_VMEM", "global load / store instructions active"),
                ("SQ_ACTIVE_INST_SCA", "scalar instructions active"))
        names = sorted(stall)
        out += ["## Where the waves' time goes (recompute path; fractions of SQ_WAVE_CYCLES)", "",
                "| counter | meaning | " + " | ".join(names) + " |",
                "|---|---|" + "---|" * len(names)]
        for c, what in rows:
            vals = [stall[n].get(c) for n in names]
            out.append(f"| {c} | {what} | " + " | ".join(
                f"{100 * sum(v) / len(v):.1f} %" if v else "-" for v in vals) + " |")
        for c in ("SQ_LDS_BANK_CONFLICT",):
            vals = [stall[n].get(c) for n in names]
            out.append(f"| {c} | LDS bank-conflict cycles (relative) | " + " | ".join(
                f"{sum(v) / len(v):.4f}" if v else "-" for v in vals) + " |")
        out.append("")
    md = os.path.join(PROFILES, "flce_qwen2_7b_head_mfma.md")
    with open(md, "w") as f:
        f.write("\n".join(out) + "\n")
    print(md)


def summarize_ceiling(prof_dir):
    """The ceiling probe's table (DIR/mfma_ceiling.txt) -> profiles/."""
    with open(os.path.join(prof_dir, "mfma_ceiling.txt")) as f:
        rows = [l.rstrip("\n") for l in f if l.startswith("|")]
    if len(rows) < 3:
        raise SystemExit("mfma_ceiling.txt holds no table")
    out = ["# Matrix-core ceiling by operand data (MI355X, no memory traffic)", "",
           "Commands ($R = repository root):", "", "```", *CEILING_COMMANDS, "```", "",
           "One 256-thread workgroup per compute unit (one wave per SIMD), each wave a 128 x 128 "
           "block of FP32 accumulators (all 256 AGPRs): 16 of v_mfma_f32_32x32x16_bf16 or 64 of "
           "v_mfma_f32_16x16x32_bf16, fed from operands held in registers (no loads, no LDS), "
           "every MFMA pairing a different operand combination; a few seconds per run. The "
           "clock column is the rate over "
           "the published 2500 TFLOP/s times 2.4 GHz: the clock the matrix cores would need "
           "at 100 % busy. The chip holds its top clock when the operand bits stay put and "
           "lowers it when they toggle: the second and third rows are about the most a bf16 "
           "contraction of such data can expect from the matrix cores on this chip (its "
           "loads, LDS traffic and other instructions draw on the same power budget).", "",
           *rows]
    md = os.path.join(PROFILES, "mfma_ceiling.md")
    with open(md, "w") as f:
        f.write("\n".join(out) + "\n")
    print(md)
    return md


def summarize_workloads(prof_dir):
    """One table over the bench lines of every workload -> profiles/."""
    rows = []
    for name in BENCH_WORKLOADS:
        path = os.path.join(prof_dir, f"bench_{name}.json")
        if not os.path.exists(path):
            continue
        lines = [l for l in open(path) if l.startswith("{")]
        if not lines:
            continue
        rows.append((name, json.loads(lines[-1])))
    gb = 1e9
    out = ["# Every workload through bench.py (MI355X, one GPU)", "",
           "Commands ($R = repository root):", "", "```", *WORKLOAD_BENCH_COMMANDS, "```", "",
           "Model basis: 6 N H V flop over all N rows; the recompute path executes 8 n H V "
           "(n valid rows), the chunked mode 6 n H V. Each workload against the dense MFMA "
           "peak of its own dtype: bf16 2500 TFLOP/s, fp32 157.3 TFLOP/s (the fp32 workload "
           "runs v_mfma_f32_32x32x2f32). PyTorch eager and hipBLASLt (bf16 only) are context, "
           "not part of the path.", "",
           "| workload | recompute ms | tokens/s | peak TFLOP/s | % peak (model) | "
           "peak extra GB | chunked ms | chunked % | PyTorch eager ms | eager peak extra GB | "
           "hipBLASLt logits GEMM ms | oracle tokens/s (host) |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, d in rows:
        ch = d.get("chunked_mode") or {}
        te = d.get("torch_eager") or {}
        vg = d.get("vendor_gemm") or {}
        cb = d.get("cpu_baseline") or {}
        pk = (BF16_PEAK if d.get("dtype") == "bf16" else F32_PEAK) / 1e12
        out.append(
            f"| {d['config']['workload']} | {d['ms_per_step']:.2f} | {d['value']:.3g} | "
            f"{pk:g} | {100 * d['mfma_frac_model']:.1f} | {d['peak_extra_bytes'] / gb:.2f} | "
            f"{ch.get('ms_per_step', float('nan')):.2f} | "
            f"{100 * ch.get('mfma_frac_model', float('nan')):.1f} | "
            f"{te.get('ms_per_step', float('nan')):.2f} | "
            f"{te.get('peak_extra_bytes', float('nan')) / gb:.1f} | "
            f"{vg.get('ms', float('nan')):.2f} | {cb.get('value', float('nan')):.0f} |")
    md = os.path.join(PROFILES, "flce_workloads_bench.md")
    with open(md, "w") as f:
        f.write("\n".join(out) + "\n")
    print(md)


def vendor_gemm(X, W, n, args, peak):
    """Reference point, not part of the path: the forward's contraction alone,
    the [n, V] logits of the valid rows materialised by torch.matmul
    (hipBLASLt), 2 n H V flop per call, no softmax."""
    import torch
    Xv = X[:n].contiguous()
    Wt = W.t()
    out = torch.empty(n, W.shape[0], dtype=X.dtype, device=X.device)
    for _ in range(max(args.warmup, 1)):
        torch.matmul(Xv, Wt, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        torch.matmul(Xv, Wt, out=out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fl = 2.0 * n * X.shape[1] * W.shape[0]
    del out
    torch.cuda.empty_cache()
    print(f"[bench] hipBLASLt logits GEMM: {ms:.3f} ms", file=sys.stderr, flush=True)
    return {"ms": ms, "tflops": fl / (ms / 1e3) / 1e12, "frac": fl / (ms / 1e3) / peak,
            "note": "torch.matmul (hipBLASLt) of the valid rows' [n, V] logits alone: the "
                    "forward's contraction without the softmax, logits materialised"}


def torch_eager(X, W, lab, w, args, peak):
    """Reference point, not part of the path: the same loss and gradients in
    PyTorch eager (F.linear + F.cross_entropy with autograd, bf16, the [N, V]
    logits and their gradient materialised), timed like the main step."""
    import torch
    import torch.nn.functional as tF
    y = lab.clone()
    if w.shift:
        y = torch.cat([y[:, 1:], torch.full_like(y[:, :1], w.ignore_index)], dim=1)
    y = y.reshape(-1)
    Xr = X.detach().requires_grad_(True)
    Wr = W.detach().requires_grad_(True)

    def step():
        loss = tF.cross_entropy(tF.linear(Xr, Wr).float(), y, ignore_index=w.ignore_index,
                                reduction=w.reduction)
        dX, dW = torch.autograd.grad(loss, (Xr, Wr))
        return loss, dX, dW

    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out = step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    del out
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    torch.cuda.empty_cache()
    print(f"[bench] torch eager: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    return {"ms_per_step": ms, "tokens_per_s": w.N / (ms / 1e3),
            "mfma_frac_model": 6.0 * w.N * w.H * w.V / (ms / 1e3) / peak,
            "peak_extra_bytes": int(peak_extra),
            "note": "PyTorch eager F.linear + F.cross_entropy (fp32 logits for the loss) with "
                    "autograd: logits and their gradient materialised"}


def chunked_mode(F, X, W, lab, w, dcode, dev, args, peak):
    """The same workload through flce_chunked (one call: loss, lse, dX, dW over
    row chunks; 6 n H V executed flop instead of 8), timed like the main step;
    reported beside the recompute path, not instead of it."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws, ws_bytes = F.chunked_workspace(w.B, w.T, w.H, w.V, dcode, dev, args.chunk_rows)

    def step():
        return F.chunked(X, W, lab, ignore_index=w.ignore_index, shift=w.shift,
                         reduction=w.reduction, ws=ws, chunk_rows=args.chunk_rows)

    out = step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    del out
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    N, H, V = w.N, w.H, w.V
    print(f"[bench] chunked mode: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    return {"ms_per_step": ms, "tokens_per_s": N / (ms / 1e3), "chunk_rows": args.chunk_rows,
            "mfma_frac_model": 6.0 * N * H * V / (ms / 1e3) / peak,
            "workspace_bytes": int(ws_bytes), "peak_extra_bytes": int(peak_extra),
            "note": "flce_chunked: gradients formed with the logits over row chunks "
                    "(bounded [C, V] slab), dW summed over chunks"}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, PROFILE_COMMANDS)
        return
    if args.summarize_workloads:
        summarize_workloads(args.summarize_workloads)
        return
    if args.summarize_ceiling:
        summarize_ceiling(args.summarize_ceiling)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_chunked:
        summarize(args.summarize_chunked, CHUNKED_PROFILE_COMMANDS, trace="prof_chunk",
                  out="flce_qwen2_7b_head_chunked_kernels.md",
                  title="Kernel time: Qwen2-7B-like LM head, chunked mode (flce_chunked)")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path "
              "has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import lm_head_linear_flce_amd as F
    import synth

    dev = torch.device("cuda:0")
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = synth.workload(args.workload)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    X = torch.from_numpy(w.X).to(dev).to(dt)
    W = torch.from_numpy(w.W).to(dev).to(dt)
    lab = torch.from_numpy(w.labels).to(dev)
    dcode = F.FLCE_DTYPE_BF16 if w.dtype == "bf16" else F.FLCE_DTYPE_F32
    n_valid = int(((lab[:, 1:] if w.shift else lab) != w.ignore_index).sum())
    peak = BF16_PEAK if w.dtype == "bf16" else F32_PEAK
    if args.vendor_gemm_only:
        print(json.dumps({"vendor_gemm": vendor_gemm(X, W, n_valid, args, peak)}), flush=True)
        return
    if args.chunked_only:
        print(json.dumps({"chunked_mode": chunked_mode(F, X, W, lab, w, dcode, dev, args,
                                                       peak)}), flush=True)
        return
    ws, ws_bytes = F.workspace(w.B, w.T, w.H, w.V, dcode, dev)
    torch.cuda.synchronize()

    def step():
        loss, lse, _, _ = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction, ws=ws)
        dX, dW, _ = F.backward(X, W, lab, lse, ignore_index=w.ignore_index, shift=w.shift,
                               reduction=w.reduction, ws=ws)
        return loss, dX, dW

    # peak extra device memory of one step (inputs already resident)
    del ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws, ws_bytes = F.workspace(w.B, w.T, w.H, w.V, dcode, dev)
    loss, dX, dW = step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    out_bytes = dX.numel() * dX.element_size() + dW.numel() * dW.element_size() + 4 * w.N
    del loss, dX, dW

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: K steps bracketed by synchronisation, with events on
    # the stream the library launches on (torch's current stream) around each
    # call: k_fwd_lse is the forward call's one GEMM launch, the k_bwd
    # launches make up the backward call (with the small prep, one-hot and
    # dX-final kernels around them, about 1 % of it; the committed kernel
    # trace lists them)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    cur = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(cur)
        loss, lse, _, _ = F.forward(X, W, lab, w.ignore_index, w.shift, w.reduction, ws=ws)
        e[1].record(cur)
        F.backward(X, W, lab, lse, ignore_index=w.ignore_index, shift=w.shift,
                   reduction=w.reduction, ws=ws)
        e[2].record(cur)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    print(f"[bench] {step_ms:.3f} ms/step: forward call {fwd_ms:.3f} ms, backward call "
          f"{bwd_ms:.3f} ms", file=sys.stderr, flush=True)
    per_kernel = {"k_fwd_lse": {"call": "flce_forward", "ms_per_step": fwd_ms},
                  "k_bwd": {"call": "flce_backward", "ms_per_step": bwd_ms}}
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms_per_step"])

    N, H, V, n = w.N, w.H, w.V, n_valid
    model_flops = 6.0 * N * H * V
    exec_flops = 8.0 * n * H * V
    t = step_ms / 1e3
    peak = BF16_PEAK if w.dtype == "bf16" else F32_PEAK
    # algorithmic flops of the dominant kernel: its contractions' 2 n H V each
    # per step over its time per step (the same ratio as per launch on average)
    ach = GEMMS_PER_STEP[dom] * 2.0 * n * H * V / (per_kernel[dom]["ms_per_step"] / 1e3)
    result = {
        "metric": METRIC,
        "value": N / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} T={w.T} N={N} H={H} V={V} {w.dtype}, "
                               f"shift={w.shift}, {w.reduction}, n_valid={n}",
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "none"},
        "mfma_frac_model": model_flops / t / peak,
        "tflops_model": model_flops / t / 1e12,
        "tflops_executed": exec_flops / t / 1e12,
        "mfma_frac_executed": exec_flops / t / peak,
        "peak_extra_bytes": int(peak_extra),
        "workspace_bytes": int(ws_bytes),
        "output_bytes": int(out_bytes),
        "logits_bytes_avoided": int(N * V * 2),
        "kernels": {k: {kk: round(vv, 4) if isinstance(vv, float) else vv
                        for kk, vv in v.items()} for k, v in per_kernel.items()},
        "roofline": {"bound": "mfma", "kernel": dom,
                     "timed": f"{per_kernel[dom]['call']} call, HIP events on its stream",
                     "achieved": ach / 1e12,
                     "peak": peak / 1e12, "unit": "TFLOP/s", "frac": ach / peak,
                     "traffic": measured_traffic(dom, w.name)},
    }
    # the measurements beside the path: each one's failure is reported in its
    # place and leaves the line intact
    def beside(key, fn):
        try:
            result[key] = fn()
        except Exception as e:  # noqa: BLE001  (reported, not swallowed)
            print(f"[bench] {key} failed: {e!r}", file=sys.stderr, flush=True)
            result[key] = {"error": repr(e)}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    if not args.no_chunked:
        beside("chunked_mode", lambda: chunked_mode(F, X, W, lab, w, dcode, dev, args, peak))
    del ws
    torch.cuda.empty_cache()
    if not args.no_vendor_gemm and w.dtype == "bf16":
        beside("vendor_gemm", lambda: vendor_gemm(X, W, n_valid, args, peak))
    if not args.no_torch_reference and w.dtype == "bf16":
        beside("torch_eager", lambda: torch_eager(X, W, lab, w, args, peak))
    if not args.no_cpu_baseline:
        print("[bench] oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = oracle_baseline(w, args.cpu_rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
