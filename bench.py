#!/usr/bin/env python3
"""Benchmark of the deterministic MoE layer on one MI355X.

One step = one pass of the whole layer on one batch of synthetic input:
routing schedule -> forward (saving the backward context) -> backward.
Default workload: bf16, T=4096 tokens, H=2048, E=64 experts, top-8, I=768,
near-uniform routing. Inputs are seeded and already resident in HBM when the
timed region starts.

Prints ONE JSON line. `value` is layer TFLOP/s: algorithmic FLOPs
(forward 6*R*H*I + backward 12*R*H*I, R = T*k routed rows, padding excluded)
divided by the measured step time.
"""
from __future__ import annotations

import argparse
import json
import os
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


# HBM traffic of the GEMM kernels, from rocprofv3 counter runs of this bench
# (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a plain copy of known
# size); valid only for the kernel sources and workload it was taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_gemm_traffic_bf16_T4096_H2048_E64_k8_I768.txt")
KERNEL_SOURCES = ["gemm_core.h", "k_gemm.hip", "k_rows.hip", "mok_device.h", "mok_launch.h", "mok_host.hip"]


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_30_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, p, minibatch_rows):
    """(bytes per launch, source) for `kernel`, or (None, reason)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.loads([ln for ln in f if ln.startswith("{")][-1])
    except (OSError, IndexError, ValueError):
        return None, "no traffic record"
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    if rec.get("workload") != p.name or rec.get("minibatch_rows") != minibatch_rows:
        return None, "counters were taken on another workload"
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None, "no record for this kernel"
    return k["bytes_per_launch"], os.path.relpath(TRAFFIC_FILE, ROOT)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=1, help="reference workload id (0-4)")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens in the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--cpu-reps", type=int, default=4,
                    help="repetitions of the CPU-baseline sample (best is reported)")
    ap.add_argument("--driver", type=int, default=0)
    ap.add_argument("--minibatch-rows", type=int, default=0)
    ap.add_argument("--ring-slots", type=int, default=0)
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only (no forward-only or MXFP8 legs); for counter runs")
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
        "reverse_combine": R * 2 * H + T * 2 * H + R * 12,       # obuf rows, dY, w/dest/dw
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
    scaled by what the same counter reads for a 1 GiB device copy, into
    TRAFFIC_FILE (text summary plus one JSON line that the bench reads)."""
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
    extra = f" --minibatch-rows {args.minibatch_rows}" if args.minibatch_rows else ""
    lines = [
        f"# HBM traffic of the grouped-GEMM and row-moving kernels: MoE layer step, bf16, {p.name} "
        f"(minibatch {mb_rows} rows)",
        "",
        "Commands (repository root on an MI355X, ROCm 7.2; one counter per run):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        f"rocprofv3 --pmc FETCH_SIZE -d <f> -o pmc -f csv -- python3 /root/repo/bench.py --steps 2 --warmup 1 --cpu-tokens 0 --only-step{extra}",
        f"rocprofv3 --pmc WRITE_SIZE -d <w> -o pmc -f csv -- python3 /root/repo/bench.py --steps 2 --warmup 1 --cpu-tokens 0 --only-step{extra}",
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
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(TRAFFIC_FILE, ROOT)}", file=sys.stderr)


def cpu_baseline(p, x, ids, w, wg, wu, wd, dy, n_tok, reps=1):
    """The fp64 oracle (as it stands) on the first n_tok tokens of the same
    workload: forward + backward, reported in the same unit."""
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
    times = []
    for _ in range(max(1, reps)):
        t0 = time.perf_counter()
        oracle.backward(xs, ids[:n_tok], w[:n_tok].astype(np.float64), Ex(), dys)   # runs forward too
        times.append(time.perf_counter() - t0)
    dt = min(times)
    flops = 18.0 * n_tok * p.k * p.H * p.I
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tok} of {p.T} tokens, forward+backward in fp64 NumPy, best of "
                      f"{len(times)} runs ({sum(times):.1f} s of CPU work in total)",
            "seconds": dt}


def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    from synthetic import CONFIGS, make_all_experts, make_dy, make_routing, make_x, router_weights

    assert torch.cuda.is_available(), "no GPU visible"
    p = CONFIGS[args.config]
    log(f"[bench] workload {p.name}: generating inputs")
    x = make_x(p)
    ids, w = make_routing(p, x)
    wg, wu, wd = make_all_experts(p, threads=16)
    dy = make_dy(p)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dx_ = dev16(x)
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    dw_ = torch.from_numpy(w).cuda()
    weights = (dev16(wg), dev16(wu), dev16(wd))
    ddy = dev16(dy)
    cfg = dict(driver=args.driver, minibatch_rows=args.minibatch_rows, ring_slots=args.ring_slots)
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=True, **cfg)
    y = torch.empty_like(dx_)
    gx = torch.empty_like(dx_)
    gwg, gwu, gwd = (torch.empty_like(t) for t in weights)
    gtw = torch.empty_like(dw_)
    stream = torch.cuda.current_stream()

    def step():
        mok.build_schedule(ws.problem, dids, ws.schedule, ws.config, stream)
        mok.forward(ws.problem, ws.schedule, dx_, dw_, weights, y, ws.workspace, ws.fwd_ctx,
                    ws.config, stream)
        mok.backward(ws.problem, ws.schedule, ws.fwd_ctx, dx_, dw_, weights, ddy, gx, gwg, gwu,
                     gwd, gtw, ws.workspace, ws.config, stream)

    def fwd_only():
        mok.build_schedule(ws.problem, dids, ws.schedule, ws.config, stream)
        mok.forward(ws.problem, ws.schedule, dx_, dw_, weights, y, ws.workspace, None, ws.config,
                    stream)

    def timed(fn, steps, trace):
        torch.cuda.synchronize()
        if trace:
            mok.trace_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        if trace:
            mok.trace_enable(False)
        stats = mok.trace_collect() if trace else {}
        return e0.elapsed_time(e1) / steps, stats

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ms_step, stats = timed(step, args.steps, trace=True)
    ms_fwd = ms_mx = ms_mxs = ms_wq = ms_rf = ms_rb = None
    mxstats = mxsstats = {}
    if not args.only_step:
        log(f"[bench] {ms_step:.3f} ms/step; forward-only timing")
        ms_fwd, _ = timed(fwd_only, args.steps, trace=True)

        # MXFP8 forward on the same workload: weights pre-quantized once
        # (outside the timed region), x quantized on the fly inside mok_forward.
        log("[bench] MXFP8 forward timing")
        wsm = F.get_workspace(p.T, p.H, p.I, p.E, p.k, dtype=mok.MOK_MXFP8, training=False, **cfg)
        qweights = F.quantize_weights(*weights)
        ymx = torch.empty_like(dx_)

        def fwd_mx():
            mok.build_schedule(wsm.problem, dids, wsm.schedule, wsm.config, stream)
            mok.forward(wsm.problem, wsm.schedule, dx_, dw_, qweights, ymx, wsm.workspace, None,
                        wsm.config, stream)

        for _ in range(2):
            fwd_mx()
        ms_mx, mxstats = timed(fwd_mx, args.steps, trace=True)
        del wsm

        # MXFP8 training step: schedule -> MXFP8 forward saving the context ->
        # MXFP8 backward. The weights (and their transposed copies for the
        # backward) are quantized before the timed region, as the pages'
        # pre-quantized weights; that quantization is timed on its own.
        log("[bench] MXFP8 step timing")
        wst = F.get_workspace(p.T, p.H, p.I, p.E, p.k, dtype=mok.MOK_MXFP8, training=True, **cfg)
        qfull = qweights + F.quantize_weights_backward(*weights)

        def step_mx():
            mok.build_schedule(wst.problem, dids, wst.schedule, wst.config, stream)
            mok.forward(wst.problem, wst.schedule, dx_, dw_, qfull, ymx, wst.workspace, wst.fwd_ctx,
                        wst.config, stream)
            mok.backward(wst.problem, wst.schedule, wst.fwd_ctx, dx_, dw_, qfull, ddy, gx, gwg, gwu, gwd,
                         gtw, wst.workspace, wst.config, stream)

        for _ in range(2):
            step_mx()
        ms_mxs, mxsstats = timed(step_mx, args.steps, trace=True)
        ms_wq, _ = timed(lambda: (F.quantize_weights(*weights), F.quantize_weights_backward(*weights)), 3,
                         trace=False)
        del wst

        # router front end on the same tokens (outside the layer step: the
        # layer takes topk_ids / topk_w as inputs)
        log("[bench] router timing")
        wr, rbias = router_weights(p)
        dwr = torch.from_numpy(np.ascontiguousarray(wr.T)).cuda()
        drb = torch.from_numpy(np.where(np.isfinite(rbias), rbias, -1e30).astype(np.float32)).cuda()
        rids, rw = torch.empty_like(dids), torch.empty_like(dw_)
        rsel, rgw = torch.empty_like(dw_), torch.empty_like(dwr)
        rg = torch.from_numpy(np.random.default_rng(p.seed + 11).standard_normal((p.T, p.k)).astype(np.float32)).cuda()

        def router_fwd():
            mok.router_forward(ws.problem, dx_, dwr, drb, rids, rw, stream)

        def router_bwd():
            mok.router_backward(ws.problem, ws.schedule, dx_, dwr, rids, rw, rg, rsel, gx, rgw, ws.config, stream)

        router_fwd()
        mok.build_schedule(ws.problem, rids, ws.schedule, ws.config, stream)
        router_bwd()
        # GPU time per call from the per-launch HIP events (back-to-back calls
        # of a ~10 us kernel are bound by the host's enqueue rate otherwise)
        _, rfstats = timed(router_fwd, args.steps, trace=True)
        _, rstats = timed(router_bwd, args.steps, trace=True)
        ms_rf = rfstats["router_forward"][1] / rfstats["router_forward"][0]
        ms_rb = rstats["router_backward"][1] / rstats["router_backward"][0]

    R, H, I = p.R, p.H, p.I
    flops_step = p.fwd_flops() + p.bwd_flops()
    value = flops_step / (ms_step * 1e-3) / 1e12

    # per-kernel live timings (HIP events on the launch stream, timed region)
    kernels = {}
    for name, (n, tot, mx) in stats.items():
        rec = {"launches_per_step": n / args.steps, "ms_per_step": tot / args.steps,
               "avg_launch_ms": tot / n}
        if name in GEMM_FLOPS_PER_ROW:
            fl = GEMM_FLOPS_PER_ROW[name] * R * H * I * args.steps
            rec["tflops"] = fl / (tot * 1e-3) / 1e12
        kernels[name] = rec
    gemms = {k: v for k, v in kernels.items() if "tflops" in v}
    dom = max(gemms, key=lambda k: gemms[k]["ms_per_step"])
    dn = stats[dom][0]
    dom_flops_per_launch = GEMM_FLOPS_PER_ROW[dom] * R * H * I * args.steps / dn
    achieved = gemms[dom]["tflops"]
    mb_rows = mok.schedule_layout(ws.problem, ws.config).minibatch_rows
    traffic, traffic_src = measured_traffic(dom, p, mb_rows)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch", "traffic_source": traffic_src,
                "flops_per_launch": dom_flops_per_launch, "avg_launch_ms": stats[dom][1] / dn}
    permute = {}
    for k, nbytes in permute_bytes(p).items():
        if k in kernels:
            kms, nl = kernels[k]["ms_per_step"], kernels[k]["launches_per_step"]
            permute[k] = {"algorithmic_gbs": round(nbytes / (kms * 1e-3) / 1e9, 1),
                          "bytes_per_step": nbytes, "ms_per_step": round(kms, 4),
                          "launches_per_step": nl}
            # counters of combine_kernel average its combine and reverse-dispatch launches
            key = "combine+reverse_dispatch" if k in ("combine", "reverse_dispatch") else k
            tb, _ = measured_traffic(key, p, mb_rows)
            if tb is not None:
                permute[k]["measured_hbm_gbs"] = round(tb * nl / (kms * 1e-3) / 1e9, 1)
    if permute:
        tot_b = sum(v["bytes_per_step"] for v in permute.values())
        tot_ms = sum(v["ms_per_step"] for v in permute.values())
        permute["all"] = {"algorithmic_gbs": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
                          "bytes_per_step": tot_b, "ms_per_step": round(tot_ms, 4),
                          "frac_of_hbm_peak": round(tot_b / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    move = sum(kernels.get(k, {}).get("ms_per_step", 0.0)
               for k in ("schedule", "gather", "combine", "reverse_combine", "reverse_dispatch"))
    gemm_ms = sum(v["ms_per_step"] for v in gemms.values())
    fwd_flops = p.fwd_flops()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"MoE SwiGLU layer fwd+bwd: {p.name}", "T": p.T, "H": H, "I": I,
                   "E": p.E, "topk": p.k, "routed_rows": R, "minibatch_rows": ws.config.minibatch_rows
                   or mok.schedule_layout(ws.problem, ws.config).minibatch_rows,
                   "ring_slots": mok.schedule_layout(ws.problem, ws.config).ring_slots,
                   "driver": {0: "default (launch-per-minibatch)", 1: "launch-per-minibatch",
                              2: "persistent (not provided)"}[args.driver]},
        "tokens_per_s": round(p.T / (ms_step * 1e-3), 1),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "gemm_tflops": round(flops_step / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
        "sched_gather_combine_share": round(move / ms_step, 4),
        "schedule_share": round(kernels.get("schedule", {}).get("ms_per_step", 0.0) / ms_step, 4),
        "kernels": kernels,
        "permute_gbs": round(permute["all"]["algorithmic_gbs"], 1) if permute else None,
        "permute": permute,
        "roofline": roofline,
    }
    if ms_fwd is not None:
        out["forward"] = {"ms": round(ms_fwd, 4), "tflops": round(fwd_flops / (ms_fwd * 1e-3) / 1e12, 2),
                          "tokens_per_s": round(p.T / (ms_fwd * 1e-3), 1)}
    if ms_mx is not None:
        out["mxfp8_forward"] = {
            "ms": round(ms_mx, 4), "tflops": round(fwd_flops / (ms_mx * 1e-3) / 1e12, 2),
            "pct_fp8_peak": round(100 * fwd_flops / (ms_mx * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
            "tokens_per_s": round(p.T / (ms_mx * 1e-3), 1),
            "gemm_tflops": {k: round(GEMM_FLOPS_PER_ROW[k] * R * H * I * args.steps / (v[1] * 1e-3) / 1e12, 2)
                            for k, v in mxstats.items() if k in GEMM_FLOPS_PER_ROW},
        }
    if ms_mxs is not None:
        out["mxfp8_step"] = {
            "ms": round(ms_mxs, 4), "tflops": round(flops_step / (ms_mxs * 1e-3) / 1e12, 2),
            "pct_fp8_peak": round(100 * flops_step / (ms_mxs * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
            "tokens_per_s": round(p.T / (ms_mxs * 1e-3), 1),
            "gemm_tflops": {k: round(GEMM_FLOPS_PER_ROW[k] * R * H * I * args.steps / (v[1] * 1e-3) / 1e12, 2)
                            for k, v in mxsstats.items() if k in GEMM_FLOPS_PER_ROW},
            "kernels_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in mxsstats.items()},
            "weight_quantize_ms": round(ms_wq, 4),
        }
    if ms_rf is not None:
        # algorithmic bytes: forward reads x and Wr once and writes ids, w;
        # backward reads ids, w, d topk_w, Wr and x, writes d_sel, dx, dWr
        # (d_sel read back once by the dWr pass)
        b_f = p.T * 2 * H + p.E * H * 4 + p.T * p.k * 8
        b_b = 2 * p.T * 2 * H + 2 * p.E * H * 4 + p.T * p.k * 20
        out["router"] = {
            "forward_ms": round(ms_rf, 4), "backward_ms": round(ms_rb, 4),
            "forward_gbs": round(b_f / (ms_rf * 1e-3) / 1e9, 1),
            "backward_gbs": round(b_b / (ms_rb * 1e-3) / 1e9, 1),
            "forward_bytes": b_f, "backward_bytes": b_b,
            "logit_tflops": round(2 * p.T * p.E * H / (ms_rf * 1e-3) / 1e12, 3),
            "timing": "HIP events around each call on the launch stream (mok_trace), averaged over the calls",
        }
    if args.cpu_tokens > 0:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(p, x, ids, w, wg, wu, wd, dy, min(args.cpu_tokens, p.T),
                                           args.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
