#!/usr/bin/env python3
"""Benchmark of the deterministic MoE layer on one MI355X.

One step = one pass of the whole layer on one batch of synthetic input:
routing schedule -> forward (saving the backward context) -> backward.
Default workload (the fwd+bwd one): bf16, T=16384 tokens, H=7168, E=32
experts, top-4, I=2048, expert loads skewed by a Zipf(0.8) routing bias.
Inputs are seeded and already resident in HBM when the timed region starts.

Prints ONE JSON line. `value` is layer TFLOP/s: algorithmic FLOPs
(forward 6*R*H*I + backward 12*R*H*I, R = T*k routed rows, padding excluded)
divided by the measured step time. The timed steps run without the library's
per-kernel tracer; per-kernel times come from a separate traced pass of the
same step. Further legs on the same line: the bf16 forward alone, the MXFP8
step on the same workload, the router front end, a 10-run bitwise
determinism check, per-expert loads, measured matrix-core and copy peaks,
the fp64 oracle timed on a sample of the workload on the host cores, and
the other workloads (bf16 forward of the small, fine-grained and Zipf(1.2)
ones; MXFP8 forward of the Zipf(1.2) one).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd/bwd TFLOP/s + tokens/s, bf16 & MXFP8; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0

# algorithmic FLOPs per routed row of each GEMM kernel, in units of H*I
GEMM_FLOPS_PER_ROW = {
    "gateup_gemm": 4, "down_gemm": 2, "bwd_dh_gemm": 2, "bwd_dwd_gemm": 2,
    "bwd_dwgu_gemm": 4, "bwd_dx_gemm": 4,
}
MOVE_KERNELS = ("schedule", "gather", "combine", "reverse_combine", "reverse_dispatch")
KERNEL_SOURCES = ["gemm_core.h", "k_gemm.hip", "k_rows.hip", "mok_device.h", "mok_launch.h", "mok_host.hip"]


def workload_tag(p):
    return f"{p.dtype}_T{p.T}_H{p.H}_E{p.E}_k{p.k}_I{p.I}"


def traffic_file(p):
    """HBM traffic record of the GEMM and row-moving kernels for workload p
    (rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this bench, scaled by a plain
    copy of known size)."""
    return os.path.join(ROOT, "profiles", f"moe_gemm_traffic_{workload_tag(p)}.txt")


def kernel_sources_sha256():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_30_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, p, minibatch_rows):
    """(bytes per launch, source) for `kernel`, or (None, reason)."""
    path = traffic_file(p)
    try:
        with open(path) as f:
            rec = json.loads([ln for ln in f if ln.startswith("{")][-1])
    except (OSError, IndexError, ValueError):
        return None, "no traffic record for this workload"
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    if rec.get("workload") != p.name or rec.get("minibatch_rows") != minibatch_rows:
        return None, "counters were taken on another workload"
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None, "no record for this kernel"
    return k["bytes_per_launch"], os.path.relpath(path, ROOT)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="workload id of the headline step (0-4)")
    ap.add_argument("--extra-configs", default="0,1,2,3",
                    help="workload ids whose forward is also timed ('' = none; 3 is the MXFP8 forward)")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens in the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--driver", type=int, default=0)
    ap.add_argument("--minibatch-rows", type=int, default=0)
    ap.add_argument("--ring-slots", type=int, default=0)
    ap.add_argument("--digest", action="store_true",
                    help="with --only-step: one more step after the timing, and the digest of its outputs "
                         "(to compare two builds bitwise)")
    ap.add_argument("--only-router", action="store_true",
                    help="the router front end only (forward and backward on the workload's tokens, "
                         "--steps calls each after one untimed call); for kernel traces")
    ap.add_argument("--router-stats-record", metavar="STATS_CSV",
                    help="write the router kernel-duration summary from a rocprofv3 --kernel-trace --stats "
                         "run of --only-router (its *_kernel_stats.csv) and exit; needs no GPU")
    ap.add_argument("--only-step", action="store_true",
                    help="the headline step only (no other legs); for counter runs")
    ap.add_argument("--step-dtype", choices=("bf16", "mxfp8"), default="bf16",
                    help="with --only-step: run the step in MXFP8 (for counter runs of the MXFP8 kernels)")
    ap.add_argument("--kernel-stats-record", metavar="STATS_CSV",
                    help="write the kernel-duration summary from a rocprofv3 --kernel-trace --stats "
                         "run of --only-step (its *_kernel_stats.csv) and exit; needs no GPU")
    ap.add_argument("--mfma-record", metavar="PMC_CSV",
                    help="write the MFMA-utilisation summary from a rocprofv3 --pmc run of --only-step "
                         "(counter_collection.csv with the counters named in the summary) and exit")
    ap.add_argument("--stall-record", nargs=2, metavar=("PMC_A_CSV", "PMC_B_CSV"),
                    help="write the stall breakdown of the GEMMs from two rocprofv3 --pmc runs of "
                         "--only-step (the counter sets named in the summary) and exit; needs no GPU")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="write the GEMM traffic record from four rocprofv3 counter_collection.csv "
                         "files (FETCH_SIZE and WRITE_SIZE of a --only-step run, then of a 1 GiB "
                         "device copy) and exit; needs no GPU")
    return ap.parse_args()


# kernel name prefixes (as rocprofv3 prints them) of the bf16 GEMM kernels and
# of the row-moving (permute) kernels; combine_kernel serves both the combine
# and the reverse-dispatch, so its record averages the two launches
GEMM_KERNEL_NAMES = {
    "gateup_kernel<false>": "gateup_gemm", "down_kernel<false>": "down_gemm",
    "bwd_dh_kernel": "bwd_dh_gemm", "bwd_dwd_kernel": "bwd_dwd_gemm",
    "bwd_dwgu_kernel": "bwd_dwgu_gemm", "bwd_dx_kernel": "bwd_dx_gemm",
    "reverse_combine_kernel": "reverse_combine",
    "::combine_kernel": "combine+reverse_dispatch",
}


def permute_bytes(p):
    """Algorithmic HBM bytes per step of the row-moving kernels (rows moved in
    + out; index and weight arrays included). The dispatch gather has no
    kernel of its own: the GEMMs read x and dY rows in place."""
    R, T, H = p.R, p.T, p.H
    return {
        "combine": R * 2 * H + R * 8 + T * 2 * H,                # obuf rows, w + dest, y rows
        "reverse_combine": R * 2 * H + T * 2 * H + R * 16,       # obuf rows, dY, w/dest/dw, w at dest
        "reverse_dispatch": R * 2 * H + R * 4 + T * 2 * H,       # dX rows, dest, dx rows
    }


def _counter_per_dispatch(path, counter):
    """{dispatch id: (kernel name, counter value)} from a counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                d = int(r["Dispatch_Id"])
                name, val = r["Kernel_Name"], float(r["Counter_Value"])
                out[d] = (name, out[d][1] + val if d in out else val)
    return out


def write_traffic_record(args):
    """Average FETCH_SIZE / WRITE_SIZE per launch of each GEMM kernel, each
    scaled by what the same counter reads for a 1 GiB device copy, into the
    workload's traffic file (text summary plus one JSON line the bench reads)."""
    import mixture_experts_layer_30_amd as mok
    from synthetic import CONFIGS
    fetch_csv, write_csv, cal_fetch_csv, cal_write_csv = args.traffic_record
    p = CONFIGS[args.config]
    cfg = mok.make_config(minibatch_rows=args.minibatch_rows, ring_slots=args.ring_slots)
    mb_rows = mok.schedule_layout(mok.make_problem(p.T, p.H, p.I, p.E, p.k), cfg).minibatch_rows
    copy_kib = float(1 << 20)

    def calib(path, counter):
        vals = [v for n, v in _counter_per_dispatch(path, counter).values() if "copyBuffer" in n]
        if not vals:
            raise SystemExit(f"{path}: no copy kernel with {counter}")
        return copy_kib / max(vals)

    ff, wf = calib(cal_fetch_csv, "FETCH_SIZE"), calib(cal_write_csv, "WRITE_SIZE")
    per = {}
    for path, counter, key in ((fetch_csv, "FETCH_SIZE", "fetch_kib"), (write_csv, "WRITE_SIZE", "write_kib")):
        for name, val in _counter_per_dispatch(path, counter).values():
            short = next((v for k, v in GEMM_KERNEL_NAMES.items() if k in name), None)
            if short:
                per.setdefault(short, {}).setdefault(key, []).append(val)
    kernels = {}
    for short in GEMM_KERNEL_NAMES.values():
        d = per.get(short, {})
        if not d.get("fetch_kib") or not d.get("write_kib"):
            continue
        fk = sum(d["fetch_kib"]) / len(d["fetch_kib"])
        wk = sum(d["write_kib"]) / len(d["write_kib"])
        kernels[short] = {"dispatches": len(d["fetch_kib"]), "fetch_kib": round(fk, 1),
                          "write_kib": round(wk, 1), "bytes_per_launch": int(round((fk * ff + wk * wf) * 1024))}
    rec = {"workload": p.name, "minibatch_rows": mb_rows, "fetch_factor": round(ff, 4),
           "write_factor": round(wf, 4), "sources_sha256": kernel_sources_sha256(), "kernels": kernels}
    extra = f" --config {args.config}" + (f" --minibatch-rows {args.minibatch_rows}" if args.minibatch_rows else "")
    bench = f"python3 /root/repo/bench.py --steps 2 --warmup 1 --cpu-tokens 0 --only-step{extra}"
    lines = [
        f"# HBM traffic of the grouped-GEMM and row-moving kernels: MoE layer step, bf16, {p.name} "
        f"(minibatch {mb_rows} rows)",
        "",
        "Commands (repository root on an MI355X, ROCm 7.2; one counter per run):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        f"rocprofv3 --pmc FETCH_SIZE -d <f> -o pmc -f csv -- {bench}",
        f"rocprofv3 --pmc WRITE_SIZE -d <w> -o pmc -f csv -- {bench}",
        "# calibration: a plain 1 GiB device copy (hipMemcpy blit kernel __amd_rocclr_copyBuffer)",
        "rocprofv3 --pmc FETCH_SIZE -d <cf> -o pmc -f csv -- python3 -c \"import torch; a=torch.ones(2**28, "
        "device='cuda', dtype=torch.int32); b=torch.empty_like(a); b.copy_(a); torch.cuda.synchronize()\"",
        "rocprofv3 --pmc WRITE_SIZE -d <cw> -o pmc -f csv -- python3 -c \"(same)\"",
        f"python3 bench.py{extra} --traffic-record <f>/pmc_counter_collection.csv <w>/pmc_counter_collection.csv "
        "<cf>/pmc_counter_collection.csv <cw>/pmc_counter_collection.csv",
        "```",
        "",
        f"Calibration: the 1 GiB copy reads FETCH_SIZE = {copy_kib / ff:.1f} KiB and WRITE_SIZE = "
        f"{copy_kib / wf:.1f} KiB, so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {wf:.4f} "
        "(the copy moves 1048576 KiB each way).",
        "",
        "Per dispatch averages over the run (3 steps, every launch of each kernel; "
        "`combine_kernel` serves both the forward combine and the backward reverse-dispatch):",
        "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
        "|---|---:|---:|---:|---:|",
    ]
    for short, k in kernels.items():
        lines.append(f"| {short} | {k['dispatches']} | {k['fetch_kib']:.0f} | {k['write_kib']:.0f} | "
                     f"{k['bytes_per_launch'] / 1e6:.1f} MB |")
    lines += ["", "Machine-readable record (bench.py reads the last line; it reports the traffic only while "
              "the kernel sources hash to `sources_sha256` and the workload matches):", "", json.dumps(rec)]
    path = traffic_file(p)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", file=sys.stderr)


def _profile_cmd(args, extra_pmc=None, trace=False):
    tail = (f"--only-step --config {args.config}" + (" --step-dtype mxfp8" if args.step_dtype == "mxfp8" else "")
            + (f" --minibatch-rows {args.minibatch_rows}" if args.minibatch_rows else ""))
    what = "--kernel-trace --stats" if trace else f"--pmc {extra_pmc}"
    steps = "--steps 5 --warmup 2" if trace else "--steps 2 --warmup 1"
    return (f"rocprofv3 {what} -d <d> -o run -f csv -- python3 /root/repo/bench.py {steps} --cpu-tokens 0 {tail}")


def _short(name):
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def write_kernel_stats_record(args):
    """Kernel durations of the step from a rocprofv3 --kernel-trace --stats
    run, as a markdown summary under profiles/."""
    import csv
    from synthetic import CONFIGS
    p = CONFIGS[args.config]
    rows = list(csv.DictReader(open(args.kernel_stats_record)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    tag = workload_tag(p) + ("_mxfp8step" if args.step_dtype == "mxfp8" else "")
    flops = {"gateup_kernel": 4, "down_kernel": 2, "bwd_dh_kernel": 2, "bwd_dwd_kernel": 2, "bwd_dwgu_kernel": 4,
             "bwd_dx_kernel": 4, "bwd_dh8_kernel": 2, "bwd_dwd8_kernel": 2, "bwd_dwgu8_kernel": 4,
             "bwd_dx8_kernel": 4}
    lines = [f"# Kernel durations: MoE layer step ({args.step_dtype}), {p.name}", "",
             "Command (repository root on an MI355X, ROCm 7.2):", "", "```", "cd /tmp && export TMPDIR=/tmp",
             _profile_cmd(args, trace=True),
             f"python3 bench.py --config {args.config}" + (" --step-dtype mxfp8" if args.step_dtype == "mxfp8" else "")
             + " --kernel-stats-record <d>/run_kernel_stats.csv", "```", "",
             "2 warm-up + 5 timed + 5 traced steps under the profiler (every launch of the run). TFLOP/s = "
             "algorithmic FLOPs per launch (routed rows only) / average duration; launches per step: "
             "gate/up and down once per ring group of minibatches, the others once.", "",
             "| kernel | calls | average ms | total ms | share | TFLOP/s per launch |", "|---|---:|---:|---:|---:|---:|"]
    rec = {}
    steps = sum(int(r["Calls"]) for r in rows if "sched_scan_kernel" in r["Name"])   # one per step
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = _short(r["Name"])
        avg = float(r["AverageNs"]) / 1e6
        key = n.split("<")[0]
        tf = ""
        if key in flops:
            nl = int(r["Calls"]) / steps               # launches per step
            tf = f"{flops[key] * p.R * p.H * p.I / nl / (avg * 1e-3) / 1e12:.1f}"
        lines.append(f"| `{n}` | {r['Calls']} | {avg:.4f} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f}% | {tf} |")
        rec[n] = {"calls": int(r["Calls"]), "avg_ms": round(avg, 5)}
    lines += ["", json.dumps({"workload": p.name, "step_dtype": args.step_dtype,
                              "sources_sha256": kernel_sources_sha256(), "kernels": rec})]
    path = os.path.join(ROOT, "profiles", f"moe_kernel_stats_{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", file=sys.stderr)


def write_router_stats_record(args):
    """Kernel durations of the router front end from a rocprofv3 --kernel-trace
    --stats run of --only-router, as a markdown summary under profiles/."""
    import csv
    from synthetic import CONFIGS
    p = CONFIGS[args.config]
    rows = [r for r in csv.DictReader(open(args.router_stats_record)) if "router" in r["Name"]]
    lines = [f"# Kernel durations: router front end, {p.name}", "",
             "Command (repository root on an MI355X, ROCm 7.2):", "", "```", "cd /tmp && export TMPDIR=/tmp",
             "rocprofv3 --kernel-trace --stats -d <d> -o run -f csv -- python3 /root/repo/bench.py --only-router "
             f"--steps 20 --config {args.config}",
             f"python3 bench.py --config {args.config} --router-stats-record <d>/run_kernel_stats.csv", "```", "",
             "One untimed call of each, then 20 forward and 20 backward calls on the workload's tokens (the "
             "router kernels only; the schedule build between them is left out). The forward is one kernel "
             "(logits, top-k, softmax); the backward two (the per-token dx rows and dWr).", "",
             "| kernel | calls | average us | total ms |", "|---|---:|---:|---:|"]
    rec = {}
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = _short(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{n}` | {r['Calls']} | {avg:.1f} | {float(r['TotalDurationNs']) / 1e6:.3f} |")
        rec[n] = {"calls": int(r["Calls"]), "avg_us": round(avg, 2)}
    lines += ["", json.dumps({"workload": p.name, "kernels": rec})]
    path = os.path.join(ROOT, "profiles", f"moe_router_kernel_stats_{workload_tag(p)}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", file=sys.stderr)


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_VALU_MFMA_BUSY_CYCLES "
                 "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def write_mfma_record(args):
    """MFMA busy share, executed vs algorithmic FLOPs and clock of each GEMM
    kernel from one rocprofv3 counter pass."""
    import csv
    from synthetic import CONFIGS
    p = CONFIGS[args.config]
    per = {}
    for r in csv.DictReader(open(args.mfma_record)):
        d = int(r["Dispatch_Id"])
        e = per.setdefault(d, {"name": r["Kernel_Name"], "dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    flops = {"gateup_kernel": 4, "down_kernel": 2, "bwd_dh_kernel": 2, "bwd_dwd_kernel": 2, "bwd_dwgu_kernel": 4,
             "bwd_dx_kernel": 4, "bwd_dh8_kernel": 2, "bwd_dwd8_kernel": 2, "bwd_dwgu8_kernel": 4,
             "bwd_dx8_kernel": 4}
    agg = {}
    steps = sum(1 for e in per.values() if "sched_scan_kernel" in e["name"])          # one per step
    for e in per.values():
        n = _short(e["name"])
        if n.split("<")[0] not in flops:
            continue
        a = agg.setdefault(n, {"n": 0, "busy": 0.0, "gui": 0.0, "mops": 0.0, "dur": 0.0})
        a["n"] += 1
        a["busy"] += e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a["gui"] += e.get("GRBM_GUI_ACTIVE", 0.0) / 8.0            # summed over the 8 XCDs
        a["mops"] += e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        a["dur"] += e["dur"]
    tag = workload_tag(p) + ("_mxfp8step" if args.step_dtype == "mxfp8" else "")
    launches = {n: a["n"] for n, a in agg.items()}
    lines = [f"# MFMA utilisation of the grouped GEMMs: MoE layer step ({args.step_dtype}), {p.name}", "",
             "Command (repository root on an MI355X, ROCm 7.2; one counter pass):", "", "```",
             "cd /tmp && export TMPDIR=/tmp", _profile_cmd(args, extra_pmc=MFMA_COUNTERS),
             f"python3 bench.py --config {args.config}" + (" --step-dtype mxfp8" if args.step_dtype == "mxfp8" else "")
             + " --mfma-record <d>/run_counter_collection.csv", "```", "",
             "Per kernel, summed over its dispatches (rocprofv3 sums each counter over its hardware "
             "instances; GRBM_GUI_ACTIVE over the 8 XCDs, so it is divided by 8):", "",
             "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs): the share of "
             "SIMD-cycles the matrix cores were busy at the clock the kernel ran;",
             "- executed GFLOP = MOPS x 512 per dispatch; algorithmic GFLOP = routed rows only; useful = "
             "algorithmic / executed;",
             "- clock = GRBM_GUI_ACTIVE per XCD / dispatch duration (timestamps of the counter run).", "",
             "| kernel | dispatches | MFMA busy | executed GFLOP | algorithmic GFLOP | useful | clock GHz |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for n, a in agg.items():
        nl = a["n"]
        ex = a["mops"] * 512 / nl / 1e9
        al = flops[n.split("<")[0]] * p.R * p.H * p.I / (launches[n] / steps) / 1e9
        busy = a["busy"] / (a["gui"] * 1024) if a["gui"] else 0.0
        clk = a["gui"] / a["dur"] if a["dur"] else 0.0
        lines.append(f"| `{n}` | {nl} | {100 * busy:.1f}% | {ex:.1f} | {al:.1f} | {100 * al / ex if ex else 0:.1f}% | "
                     f"{clk:.2f} |")
    path = os.path.join(ROOT, "profiles", f"moe_gemm_mfma_util_{tag}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", file=sys.stderr)


STALL_COUNTERS_A = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
                    "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE")
STALL_COUNTERS_B = ("SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM_RD "
                    "SQ_LDS_DATA_FIFO_FULL SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU TA_TA_BUSY "
                    "TA_DATA_STALLED_BY_TC_CYCLES TCP_TCC_READ_REQ_LATENCY TCP_TCC_READ_REQ "
                    "TCP_PENDING_STALL_CYCLES TCP_READ_TAGCONFLICT_STALL_CYCLES GRBM_GUI_ACTIVE")
GEMM_PREFIXES = ("gateup_kernel", "down_kernel", "bwd_dh", "bwd_dwd", "bwd_dwgu", "bwd_dx")


def _pmc_per_kernel(path):
    """Counters of one rocprofv3 --pmc csv, summed per kernel over its
    dispatches (each counter summed over its hardware instances)."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        e = per.setdefault(d, {"name": _short(r["Kernel_Name"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = {}
    for e in per.values():
        if not e["name"].startswith(GEMM_PREFIXES):
            continue
        a = agg.setdefault(e["name"], {"n": 0})
        a["n"] += 1
        for k, v in e.items():
            if k != "name":
                a[k] = a.get(k, 0.0) + v
    return agg


def write_stall_record(args):
    """Where the GEMM wavefronts and their memory path spend their cycles,
    from two rocprofv3 counter passes of the step."""
    from synthetic import CONFIGS
    p = CONFIGS[args.config]
    A, B = (_pmc_per_kernel(f) for f in args.stall_record)
    tag = workload_tag(p) + ("_mxfp8step" if args.step_dtype == "mxfp8" else "")
    dt = " --step-dtype mxfp8" if args.step_dtype == "mxfp8" else ""
    lines = [f"# Stall breakdown of the grouped GEMMs: MoE layer step ({args.step_dtype}), {p.name}", "",
             "Commands (repository root on an MI355X, ROCm 7.2; two counter passes, each a run of its own):",
             "", "```", "cd /tmp && export TMPDIR=/tmp",
             _profile_cmd(args, extra_pmc=STALL_COUNTERS_A).replace("<d>", "<a>"),
             _profile_cmd(args, extra_pmc=STALL_COUNTERS_B).replace("<d>", "<b>"),
             f"python3 bench.py --config {args.config}{dt} --stall-record <a>/run_counter_collection.csv "
             "<b>/run_counter_collection.csv", "```", "",
             f"Kernel sources sha256: `{kernel_sources_sha256()}`", "",
             "Per kernel, summed over its dispatches; GRBM_GUI_ACTIVE is summed over the 8 XCDs and divided "
             "by 8. Wave shares are of SQ_WAVE_CYCLES (cycles summed over resident waves); unit shares are of "
             "the kernel's busy cycles times 256 units (one texture address unit and one L1 per CU):", "",
             "- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x 1024 SIMDs);",
             "- wait any / wait inst / wait LDS: SQ_WAIT_ANY, SQ_WAIT_INST_ANY (waiting on an instruction's "
             "inputs), SQ_WAIT_INST_LDS;",
             "- VMEM active / LDS active: SQ_ACTIVE_INST_VMEM, SQ_ACTIVE_INST_LDS;",
             "- bank conflicts per LDS instruction: SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS;",
             "- TA busy, TA stalled by L1: TA_TA_BUSY, TA_DATA_STALLED_BY_TC_CYCLES;",
             "- L2 read latency (cycles): TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ; L1 pending stall: "
             "TCP_PENDING_STALL_CYCLES;",
             "- VMEM loads in flight per wave: SQ_INST_LEVEL_VMEM / SQ_INSTS_VMEM_RD.", "",
             "| kernel | dispatches | MFMA busy | wait any | wait inst | wait LDS | VMEM active | LDS active "
             "| conflicts / LDS inst | TA busy | TA stalled | L2 latency | L1 pending | VMEM in flight |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for n, a in A.items():
        b = B.get(n)
        if b is None:
            continue
        gui_a, gui_b, wc = a["GRBM_GUI_ACTIVE"] / 8, b["GRBM_GUI_ACTIVE"] / 8, a["SQ_WAVE_CYCLES"]
        pct = lambda v, d: f"{100 * v / d:.1f}%" if d else "-"   # noqa: E731
        lines.append(
            f"| `{n}` | {a['n']:.0f} | {pct(a['SQ_VALU_MFMA_BUSY_CYCLES'], gui_a * 1024)} "
            f"| {pct(a['SQ_WAIT_ANY'], wc)} | {pct(a['SQ_WAIT_INST_ANY'], wc)} | {pct(a['SQ_WAIT_INST_LDS'], wc)} "
            f"| {pct(a['SQ_ACTIVE_INST_VMEM'], wc)} | {pct(a['SQ_ACTIVE_INST_LDS'], wc)} "
            f"| {b['SQ_LDS_BANK_CONFLICT'] / max(b['SQ_INSTS_LDS'], 1):.2f} "
            f"| {pct(b['TA_TA_BUSY'], gui_b * 256)} | {pct(b['TA_DATA_STALLED_BY_TC_CYCLES'], gui_b * 256)} "
            f"| {b['TCP_TCC_READ_REQ_LATENCY'] / max(b['TCP_TCC_READ_REQ'], 1):.0f} "
            f"| {pct(b['TCP_PENDING_STALL_CYCLES'], gui_b * 256)} "
            f"| {b['SQ_INST_LEVEL_VMEM'] / max(b['SQ_INSTS_VMEM_RD'], 1):.1f} |")
    path = os.path.join(ROOT, "profiles", f"moe_gemm_stalls_{tag}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}", file=sys.stderr)


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(p, x, ids, w, wg, wu, wd, dy, n_tok):
    """The fp64 oracle (as it stands) on the first n_tok tokens of the same
    workload: the schedule of the whole batch, then forward and forward +
    backward of the sample, each timed on its own."""
    import numpy as np
    import oracle
    from synthetic import bf16_to_f32
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=os.cpu_count())
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()

    class Ex:
        def __len__(self):
            return p.E

        def __getitem__(self, e):
            return tuple(bf16_to_f32(m[e]).astype(np.float64) for m in (wg, wu, wd))

    xs = bf16_to_f32(x[:n_tok]).astype(np.float64)
    dys = bf16_to_f32(dy[:n_tok]).astype(np.float64)
    ws = w[:n_tok].astype(np.float64)
    t0 = time.perf_counter()
    oracle.schedule(ids, p.E)
    t1 = time.perf_counter()
    oracle.forward(xs, ids[:n_tok], ws, Ex())
    t2 = time.perf_counter()
    oracle.backward(xs, ids[:n_tok], ws, Ex(), dys)      # recomputes the forward itself
    t3 = time.perf_counter()
    flops = 18.0 * n_tok * p.k * p.H * p.I
    return {"value": flops / (t3 - t2) / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tok} of {p.T} tokens of the same workload: forward + backward in fp64 NumPy "
                      f"(oracle.backward, which also runs the forward), one run; "
                      f"{t1 - t0 + t3 - t1:.1f} s of CPU work in total",
            "seconds_schedule_full_batch": round(t1 - t0, 3), "seconds_forward": round(t2 - t1, 3),
            "seconds_forward_backward": round(t3 - t2, 3),
            "seconds_backward_only": round((t3 - t2) - (t2 - t1), 3), "tokens": n_tok}


# ------------------------------------------------------------------ timing helpers
def time_steps(fn, steps, stream):
    """(mean, median, min) ms of `steps` calls of fn, each bracketed by events
    on the launch stream; synchronized before and after."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, statistics.median(per), min(per)


def traced(fn, steps):
    """Per-kernel {name: (launches, total_ms, max_ms)} over `steps` calls, from
    the library's per-launch HIP events (a separate pass from the timed one)."""
    import torch
    import mixture_experts_layer_30_amd as mok
    torch.cuda.synchronize()
    mok.trace_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    mok.trace_enable(False)
    return mok.trace_collect()


def gemm_rates(stats, p, steps):
    return {k: round(GEMM_FLOPS_PER_ROW[k] * p.R * p.H * p.I * steps / (v[1] * 1e-3) / 1e12, 2)
            for k, v in stats.items() if k in GEMM_FLOPS_PER_ROW}


def load_stats(ids, E):
    import numpy as np
    c = np.bincount(ids.reshape(-1)[(ids.reshape(-1) >= 0) & (ids.reshape(-1) < E)], minlength=E)
    return {"experts": E, "rows": int(c.sum()), "mean": round(float(c.mean()), 1), "max": int(c.max()),
            "min": int(c.min()), "empty": int((c == 0).sum()), "max_over_mean": round(float(c.max() / c.mean()), 3),
            "cv": round(float(c.std() / c.mean()), 3)}


def digest(tensors):
    """Two integer checksums per tensor (sum, and position-weighted sum, of
    its 32-bit words; exact integer arithmetic on the device) and their sha256."""
    import torch
    parts = []
    for t in tensors:
        v = t.contiguous().view(torch.int32).reshape(-1).to(torch.int64)
        wgt = torch.arange(v.numel(), device=v.device, dtype=torch.int64) % 65521 + 1
        parts += [int(v.sum().item()), int((v * wgt).sum().item())]
    return parts, hashlib.sha256(json.dumps(parts).encode()).hexdigest()[:16]


def measure_peaks(stream):
    """Matrix-core rate of back-to-back MFMAs on register operands (bf16 and
    MXFP8), and device copy bandwidth (read + write bytes of a 4 GiB copy)."""
    import torch
    import mixture_experts_layer_30_amd as mok
    out = {}
    wgs = 256 * 8
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    for kind, name, iters in ((0, "bf16_tflops", 2000), (1, "fp8_tflops", 1000)):
        fl = mok.probe_mfma(kind, wgs, 50, sink, stream)
        fl = 0.0
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fl = mok.probe_mfma(kind, wgs, iters, sink, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name] = round(fl / (best * 1e-3) / 1e12, 1)
    a = torch.empty(1 << 30, dtype=torch.int32, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    out["copy_gbs"] = round(2 * a.numel() * 4 / (best * 1e-3) / 1e9, 1)
    out["how"] = ("mok_probe_mfma: 2048 workgroups x 4 wavefronts, 8 MFMA chains each, best of 3; "
                  "copy: torch copy_ of a 4 GiB buffer (read + write bytes), best of 3")
    return out


# ------------------------------------------------------------------ workloads on the device
class Dev:
    """Device copies of a workload's inputs."""

    def __init__(self, p, threads=16, with_dy=True):
        import numpy as np
        import torch
        from synthetic import make_all_experts, make_dy, make_routing, make_x
        self.p = p
        t0 = time.time()
        self.x_h = make_x(p)
        self.ids_h, self.w_h = make_routing(p, self.x_h)
        self.wg_h, self.wu_h, self.wd_h = make_all_experts(p, threads=threads)
        self.dy_h = make_dy(p) if with_dy else None
        log(f"[bench] {p.name}: inputs generated in {time.time() - t0:.1f} s")

        def dev16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        self.x = dev16(self.x_h)
        self.ids = torch.from_numpy(self.ids_h.astype(np.int32)).cuda()
        self.w = torch.from_numpy(self.w_h).cuda()
        self.weights = (dev16(self.wg_h), dev16(self.wu_h), dev16(self.wd_h))
        self.dy = dev16(self.dy_h) if with_dy else None


def forward_leg(d, dtype, steps, warmup, stream, cfg):
    """Schedule + forward (no context) of workload d; bf16 or MXFP8."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = d.p
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, dtype=dtype, training=False, **cfg)
    wts = d.weights if dtype == mok.MOK_BF16 else F.quantize_weights(*d.weights)
    y = torch.empty_like(d.x)

    def fwd():
        mok.build_schedule(ws.problem, d.ids, ws.schedule, ws.config, stream)
        mok.forward(ws.problem, ws.schedule, d.x, d.w, wts, y, ws.workspace, None, ws.config, stream)

    for _ in range(warmup):
        fwd()
    mean, med, mn = time_steps(fwd, steps, stream)
    st = traced(fwd, steps)
    fl = p.fwd_flops()
    peak = PEAK_BF16_TFLOPS if dtype == mok.MOK_BF16 else PEAK_FP8_TFLOPS
    move = sum(st[k][1] for k in MOVE_KERNELS if k in st) / steps
    sched = st["schedule"][1] / steps if "schedule" in st else 0.0
    traced_ms = sum(v[1] for v in st.values()) / steps
    rec = {"workload": p.name, "dtype": "mxfp8" if dtype == mok.MOK_MXFP8 else "bf16",
           "ms": round(mean, 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
           "tflops": round(fl / (mean * 1e-3) / 1e12, 2),
           "pct_peak": round(100 * fl / (mean * 1e-3) / 1e12 / peak, 2),
           "tokens_per_s": round(p.T / (mean * 1e-3), 1),
           "gemm_tflops": gemm_rates(st, p, steps),
           "schedule_share": round(sched / traced_ms, 4) if traced_ms else None,
           "sched_gather_combine_share": round(move / traced_ms, 4) if traced_ms else None,
           "minibatch_rows": mok.schedule_layout(ws.problem, ws.config).minibatch_rows,
           "loads": load_stats(d.ids_h, p.E)}
    del ws, wts, y
    return rec


def forward_drivers(d, steps, warmup, stream):
    """Schedule + forward (bf16, no context) of workload d under the three
    drivers: one launch per stage per ring group (driver 1), the persistent
    minibatch kernel (driver 2, two calls), and the single launch
    (mok_forward_fused). Results are bitwise the same (GPU tests)."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = d.p
    y = torch.empty_like(d.x)
    rec = {"workload": p.name}
    for name, drv in (("launch_per_stage", 1), ("persistent", 2), ("single_launch", None)):
        ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=False, driver=drv or 0)

        def fwd():
            if drv is None:
                mok.forward_fused(ws.problem, d.ids, ws.schedule, d.x, d.w, d.weights, y, ws.workspace, None,
                                  ws.config, stream)
            else:
                mok.build_schedule(ws.problem, d.ids, ws.schedule, ws.config, stream)
                mok.forward(ws.problem, ws.schedule, d.x, d.w, d.weights, y, ws.workspace, None, ws.config,
                            stream)

        for _ in range(warmup):
            fwd()
        mean, med, mn = time_steps(fwd, steps, stream)
        rec[name] = {"ms": round(mean, 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
                     "tflops": round(p.fwd_flops() / (mean * 1e-3) / 1e12, 2)}
        del ws
    return rec



def router_leg(d, p, K, stream, cfg, gx):
    """Router front end on the workload's tokens (outside the layer step: the
    layer takes topk_ids / topk_w as inputs): forward and backward, per-call
    time from the library tracer's HIP events."""
    import numpy as np
    import torch

    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    from synthetic import router_weights
    H = p.H
    wr, rbias = router_weights(p)
    dwr = torch.from_numpy(np.ascontiguousarray(wr.T)).cuda()
    drb = torch.from_numpy(np.where(np.isfinite(rbias), rbias, -1e30).astype(np.float32)).cuda()
    rids, rw = torch.empty_like(d.ids), torch.empty_like(d.w)
    rsel, rgw = torch.empty_like(d.w), torch.empty_like(dwr)
    rg = torch.from_numpy(np.random.default_rng(p.seed + 11).standard_normal((p.T, p.k)).astype(np.float32)).cuda()
    wsr = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=False, **cfg)
    prob = mok.make_problem(p.T, p.H, p.I, p.E, p.k)

    def router_fwd():
        mok.router_forward(prob, d.x, dwr, drb, rids, rw, stream)

    def router_bwd():
        mok.router_backward(prob, wsr.schedule, d.x, dwr, rids, rw, rg, rsel, gx, rgw, wsr.config, stream)

    router_fwd()
    mok.build_schedule(wsr.problem, rids, wsr.schedule, wsr.config, stream)
    router_bwd()
    rfst, rbst = traced(router_fwd, K), traced(router_bwd, K)
    ms_rf = rfst["router_forward"][1] / rfst["router_forward"][0]
    ms_rb = rbst["router_backward"][1] / rbst["router_backward"][0]
    b_f = p.T * 2 * H + p.E * H * 4 + p.T * p.k * 8
    b_b = 2 * p.T * 2 * H + 2 * p.E * H * 4 + p.T * p.k * 20
    return {
        "workload": p.name, "forward_ms": round(ms_rf, 4), "backward_ms": round(ms_rb, 4),
        "forward_gbs": round(b_f / (ms_rf * 1e-3) / 1e9, 1), "backward_gbs": round(b_b / (ms_rb * 1e-3) / 1e9, 1),
        "forward_bytes": b_f, "backward_bytes": b_b,
        "logit_tflops": round(2 * p.T * p.E * H / (ms_rf * 1e-3) / 1e12, 3),
        "timing": "HIP events around each call on the launch stream (mok_trace), averaged over the calls"}

def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(args)
        return
    if args.stall_record:
        write_stall_record(args)
        return
    if args.kernel_stats_record:
        write_kernel_stats_record(args)
        return
    if args.router_stats_record:
        write_router_stats_record(args)
        return
    if args.mfma_record:
        write_mfma_record(args)
        return
    if args.step_dtype == "mxfp8" and not args.only_step:
        raise SystemExit("--step-dtype mxfp8 is for counter runs: use it with --only-step")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    from synthetic import CONFIGS

    assert torch.cuda.is_available(), "no GPU visible"
    mok.lib()
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    cfg = dict(driver=args.driver, minibatch_rows=args.minibatch_rows, ring_slots=args.ring_slots)

    peaks = None
    if not args.only_step and not args.only_router:
        log("[bench] measured peaks (matrix cores, copy)")
        peaks = measure_peaks(stream)
        log(f"[bench] {peaks}")

    p = CONFIGS[args.config]
    d = Dev(p)
    if args.only_router:
        rr = router_leg(d, p, K, stream, cfg, torch.empty_like(d.x))
        print(json.dumps({"router": rr, "steps": K}))
        return
    mx_step = args.step_dtype == "mxfp8"
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=True,
                         dtype=mok.MOK_MXFP8 if mx_step else mok.MOK_BF16, **cfg)
    step_w = (F.quantize_weights(*d.weights) + F.quantize_weights_backward(*d.weights)) if mx_step else d.weights
    y = torch.empty_like(d.x)
    gx = torch.empty_like(d.x)
    gwg, gwu, gwd = (torch.empty_like(t) for t in d.weights)
    gtw = torch.empty_like(d.w)
    outs = (y, gx, gwg, gwu, gwd, gtw)

    def step():
        mok.build_schedule(ws.problem, d.ids, ws.schedule, ws.config, stream)
        mok.forward(ws.problem, ws.schedule, d.x, d.w, step_w, y, ws.workspace, ws.fwd_ctx, ws.config, stream)
        mok.backward(ws.problem, ws.schedule, ws.fwd_ctx, d.x, d.w, step_w, d.dy, gx, gwg, gwu, gwd, gtw,
                     ws.workspace, ws.config, stream)

    log(f"[bench] warmup {W} steps")
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {K} steps (tracer off)")
    ms_step, ms_med, ms_min = time_steps(step, K, stream)
    log(f"[bench] {ms_step:.3f} ms/step (median {ms_med:.3f}, min {ms_min:.3f}); traced pass")
    stats = traced(step, K)

    R, H, I = p.R, p.H, p.I
    flops_step = p.fwd_flops() + p.bwd_flops()
    value = flops_step / (ms_step * 1e-3) / 1e12
    kernels = {}
    for name, (n, tot, mx) in stats.items():
        rec = {"launches_per_step": n / K, "ms_per_step": round(tot / K, 4), "avg_launch_ms": round(tot / n, 4)}
        if name in GEMM_FLOPS_PER_ROW:
            rec["tflops"] = round(GEMM_FLOPS_PER_ROW[name] * R * H * I * K / (tot * 1e-3) / 1e12, 2)
        kernels[name] = rec
    traced_ms = sum(v[1] for v in stats.values()) / K
    gemms = {k: v for k, v in kernels.items() if "tflops" in v}
    dom = max(gemms, key=lambda k: gemms[k]["ms_per_step"])
    dn = stats[dom][0]
    dom_flops_per_launch = GEMM_FLOPS_PER_ROW[dom] * R * H * I * K / dn
    dom_avg_ms = stats[dom][1] / dn
    achieved = dom_flops_per_launch / (dom_avg_ms * 1e-3) / 1e12
    mb_rows = mok.schedule_layout(ws.problem, ws.config).minibatch_rows
    traffic, traffic_src = measured_traffic(dom, p, mb_rows)
    peak = PEAK_FP8_TFLOPS if mx_step else PEAK_BF16_TFLOPS
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch", "traffic_source": traffic_src,
                "flops_per_launch": dom_flops_per_launch, "avg_launch_ms": round(dom_avg_ms, 5),
                "timing": "HIP events around each launch on the launch stream (library tracer), separate pass"}
    if peaks:
        roofline["frac_of_measured_mfma_peak"] = round(achieved / peaks["bf16_tflops"], 4)
    permute = {}
    for k, nbytes in permute_bytes(p).items():
        if k in kernels:
            kms, nl = kernels[k]["ms_per_step"], kernels[k]["launches_per_step"]
            permute[k] = {"algorithmic_gbs": round(nbytes / (kms * 1e-3) / 1e9, 1), "bytes_per_step": nbytes,
                          "ms_per_step": round(kms, 4), "launches_per_step": nl}
            key = "combine+reverse_dispatch" if k in ("combine", "reverse_dispatch") else k
            tb, _ = measured_traffic(key, p, mb_rows)
            if tb is not None:
                permute[k]["measured_hbm_gbs"] = round(tb * nl / (kms * 1e-3) / 1e9, 1)
    if permute:
        tot_b = sum(v["bytes_per_step"] for v in permute.values())
        tot_ms = sum(v["ms_per_step"] for v in permute.values())
        permute["all"] = {"algorithmic_gbs": round(tot_b / (tot_ms * 1e-3) / 1e9, 1), "bytes_per_step": tot_b,
                          "ms_per_step": round(tot_ms, 4),
                          "frac_of_hbm_peak": round(tot_b / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if peaks:
            permute["all"]["frac_of_measured_copy"] = round(tot_b / (tot_ms * 1e-3) / 1e9 / peaks["copy_gbs"], 4)
    move = sum(kernels.get(k, {}).get("ms_per_step", 0.0) for k in MOVE_KERNELS)
    gemm_ms = sum(v["ms_per_step"] for v in gemms.values())
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8" if mx_step else "bf16",
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": f"MoE SwiGLU layer fwd+bwd, bf16: {p.name}", "T": p.T, "H": H, "I": I,
                   "E": p.E, "topk": p.k, "routed_rows": R, "minibatch_rows": mb_rows,
                   "ring_slots": mok.schedule_layout(ws.problem, ws.config).ring_slots,
                   "driver": {0: "default (launch per stage per ring group)", 1: "launch per stage per ring group",
                              2: "persistent"}[args.driver]},
        "ms_per_step_median": round(ms_med, 4), "ms_per_step_min": round(ms_min, 4),
        "tokens_per_s": round(p.T / (ms_step * 1e-3), 1),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "gemm_tflops": round(flops_step / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
        "sched_gather_combine_share": round(move / traced_ms, 4),
        "schedule_share": round(kernels.get("schedule", {}).get("ms_per_step", 0.0) / traced_ms, 4),
        "kernels": kernels,
        "permute_gbs": permute["all"]["algorithmic_gbs"] if permute else None,
        "permute": permute,
        "roofline": roofline,
        "loads": load_stats(d.ids_h, p.E),
    }
    if peaks:
        out["measured_peaks"] = peaks
        out["pct_measured_bf16_peak"] = round(100 * value / peaks["bf16_tflops"], 2)

    # 10 runs of the step on the same buffers: every output bitwise equal
    # (left out of counter runs, which time the step only)
    log("[bench] determinism: 10 runs")
    ref = None
    same = True
    dig = None
    for run in range(0 if args.only_step else 10):
        for o in outs:
            o.fill_(7)
        step()
        torch.cuda.synchronize()
        parts, h = digest(outs)
        if ref is None:
            ref, dig = parts, h
        same = same and parts == ref
    if not args.only_step:
        out["determinism"] = {"runs": 10, "bitwise_identical": same, "digest": dig,
                              "outputs": "y, dx, dWg, dWu, dWd, d topk_w"}
    elif args.digest:
        for o in outs:
            o.fill_(7)
        step()
        torch.cuda.synchronize()
        out["digest"] = {"digest": digest(outs)[1], "outputs": "y, dx, dWg, dWu, dWd, d topk_w"}

    if not args.only_step:
        log("[bench] forward-only timing")
        out["forward"] = forward_leg(d, mok.MOK_BF16, K, W, stream, cfg)
        del ws
        log("[bench] forward drivers (schedule + forward)")
        out["forward_drivers"] = forward_drivers(d, K, W, stream)
        # MXFP8 step on the same workload: the weights (and their transposed
        # copies for the backward) are quantized once before the timed region,
        # as the pages' pre-quantized weights; that quantization is timed too.
        log("[bench] MXFP8 step timing")
        wst = F.get_workspace(p.T, p.H, p.I, p.E, p.k, dtype=mok.MOK_MXFP8, training=True, **cfg)
        t_q = time_steps(lambda: F.quantize_weights(*d.weights) + F.quantize_weights_backward(*d.weights), 3,
                         stream)[0]
        qfull = F.quantize_weights(*d.weights) + F.quantize_weights_backward(*d.weights)
        ymx = torch.empty_like(d.x)

        def step_mx():
            mok.build_schedule(wst.problem, d.ids, wst.schedule, wst.config, stream)
            mok.forward(wst.problem, wst.schedule, d.x, d.w, qfull, ymx, wst.workspace, wst.fwd_ctx, wst.config,
                        stream)
            mok.backward(wst.problem, wst.schedule, wst.fwd_ctx, d.x, d.w, qfull, d.dy, gx, gwg, gwu, gwd, gtw,
                         wst.workspace, wst.config, stream)

        for _ in range(W):
            step_mx()
        mxm, mxmed, mxmin = time_steps(step_mx, K, stream)
        mxst = traced(step_mx, K)
        out["mxfp8_step"] = {
            "workload": p.name, "ms": round(mxm, 4), "ms_median": round(mxmed, 4), "ms_min": round(mxmin, 4),
            "tflops": round(flops_step / (mxm * 1e-3) / 1e12, 2),
            "pct_fp8_peak": round(100 * flops_step / (mxm * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
            "tokens_per_s": round(p.T / (mxm * 1e-3), 1), "gemm_tflops": gemm_rates(mxst, p, K),
            "kernels_ms_per_step": {k: round(v[1] / K, 4) for k, v in mxst.items()},
            "weight_quantize_ms": round(t_q, 4)}
        if peaks:
            out["mxfp8_step"]["pct_measured_fp8_peak"] = round(
                100 * flops_step / (mxm * 1e-3) / 1e12 / peaks["fp8_tflops"], 2)
        del wst, qfull, ymx

        # router front end on the same tokens (outside the layer step: the
        # layer takes topk_ids / topk_w as inputs)
        log("[bench] router timing")
        out["router"] = router_leg(d, p, K, stream, cfg, gx)

    if args.cpu_tokens > 0:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(p, d.x_h, d.ids_h, d.w_h, d.wg_h, d.wu_h, d.wd_h, d.dy_h,
                                           min(args.cpu_tokens, p.T))

    extra = [int(c) for c in args.extra_configs.split(",") if c.strip()] if not args.only_step else []
    if extra:
        del d, outs, y, gx, gwg, gwu, gwd, gtw
        torch.cuda.empty_cache()
        out["configs"] = {}
        cache = {}
        for c in extra:
            q = CONFIGS[c]
            key = (q.T, q.H, q.E, q.k, q.I, q.seed, q.zipf_s, q.empty_den)
            if key not in cache:
                cache.clear()
                torch.cuda.empty_cache()
                cache[key] = Dev(q, with_dy=False)
            dq = cache[key]
            dq.p = q
            log(f"[bench] workload {c}: {q.name}")
            out["configs"][str(c)] = forward_leg(dq, mok.MOK_MXFP8 if q.dtype == "mxfp8" else mok.MOK_BF16,
                                                 K, W, stream, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
