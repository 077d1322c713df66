#!/usr/bin/env python3
"""Benchmark of one quantized-momentum Muon step on one MI355X.

Default workload: the Llama-8B-shaped layer (q/o 4096x4096, k/v 1024x4096,
gate/up 14336x4096, down 4096x14336), bf16 grads ~N(0, 1e-3), int8 momentum
state, one norm group per matrix; a step is the full Muon step: q8 update +
group norms (qmuon_update_normalize_groups), then quintic Newton-Schulz
(T = 5, bf16 MFMA) of every matrix with the weight update fused into its last
product (muon_apply).  muon_step is exactly these two calls; they are issued
separately here so HIP events on the launch stream time each phase live.

Printed: one JSON line.  value = q8 update GB/s (algorithmic bytes: int8
codes read+write, bf16 grad read+write, fp32 absmax read+write per 256
elements = 6.03125 B/element); ns_tflops = NS TFLOP/s (algorithmic FLOPs with
the two symmetric products at lower-triangle cost); `roofline` is for the
dominant kernel (the NS products, MFMA bound), `roofline_update` for the HBM-
bound update kernel; `cpu_baseline` times the CPU oracle on a bounded sample.

Other workloads (not the headline): --workload layerset28 (the 28-layer
2048-hidden set, grouped update + normalisation only), --workload muonbp
(4096x14336, 8 column blocks, P = 5).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "q8 momentum update GB/s (%HBM peak) + Newton-Schulz TFLOP/s (%MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_PEAK_TFLOPS = 157.3
BYTES_PER_ELEM_UPDATE = 6.03125      # 1+1 code, 2+2 bf16 grad, 8/256 absmax
BYTES_PER_ELEM_SCALE = 4.0           # bf16 grad read + write (normalise pass)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "layerset28", "muonbp"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ref-copy-mib", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB once (a kernel of "
                         "known traffic, to calibrate HBM byte counters in a profiler run)")
    return ap.parse_args()


def ns_sym_flops(rows, cols, steps):
    m, n = min(rows, cols), max(rows, cols)
    return steps * (n * m * (m + 1) + m * m * (m + 1) + 2 * m * m * n)


def cpu_baseline(host_q, host_ns, steps):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from oracle import ns
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count()
    codes, absmax, grad = host_q
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.q8_update(codes, absmax, grad, 0.95, oracle.BF16)
        reps += 1
        if time.perf_counter() - t0 > 5.0 or reps >= 20:
            break
    t_q = (time.perf_counter() - t0) / reps
    gbs = codes.size * BYTES_PER_ELEM_UPDATE / t_q / 1e9
    x = host_ns
    t0 = time.perf_counter()
    ns.ns_orthogonalize(x, steps)
    t_ns = time.perf_counter() - t0
    fl = ns_sym_flops(x.shape[0], x.shape[1], steps)
    return {
        "value": round(gbs, 3), "unit": "GB/s", "cores": max(oracle.num_threads(), blas_threads),
        "kind": "oracle",
        "sample": (f"q8 update of one {codes.size}-element bf16 tensor (C oracle, {reps} reps) + "
                   f"fp64 NS T={steps} of one {x.shape[0]}x{x.shape[1]} matrix (numpy oracle)"),
        "ns_tflops": round(fl / t_ns / 1e12, 5),
        "q8_seconds": round(t_q, 4), "ns_seconds": round(t_ns, 3),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_momentum_newton_amd as q
    from harness import inputs as H
    dev = "cuda"
    torch.cuda.init()

    if args.workload == "llama8b":
        tensors, segments, ng = H.config3_layout()
    elif args.workload == "layerset28":
        tensors, segments, ng = H.config2_layout()
    else:
        cfg = H.config4_shape()
        tensors = [("w", cfg["rows"], cfg["cols"])]
        segments, ng = [(0, 0, cfg["rows"] * cfg["cols"], 0)], 1
    seed = {"llama8b": 1003, "layerset28": 1002, "muonbp": 1004}[args.workload]
    trip, mats, numel = [], [], 0
    for i, (name, r, c) in enumerate(tensors):
        codes, absmax = H.prior_state(r * c, dev, seed, i)
        g = H.grad((r, c), torch.bfloat16, dev, seed, i,
                   outlier_frac=0.01 if args.workload == "layerset28" else 0.0).reshape(-1)
        trip.append((codes, absmax, g))
        if args.workload != "layerset28":
            w = H.weights((r, c), dev, seed, i)
            if args.workload == "muonbp":
                mats.append((r, c, cfg["block_rows"], cfg["block_cols"], w))
            else:
                mats.append((r, c, r, c, w))
        numel += r * c
    torch.cuda.synchronize()
    host_q = None
    if not args.no_cpu_baseline:
        import numpy as np
        k = min(range(len(tensors)), key=lambda i: abs(tensors[i][1] * tensors[i][2] - 16 * 2 ** 20))
        host_q = (trip[k][0].cpu().numpy(), trip[k][1].cpu().numpy(),
                  trip[k][2].view(torch.int16).cpu().numpy().view(np.uint16))
        kn = min(range(len(tensors)), key=lambda i: tensors[i][1] * tensors[i][2])
        host_ns = trip[kn][2].float().cpu().numpy().astype(np.float64).reshape(
            tensors[kn][1], tensors[kn][2])

    plan = q.Plan(trip, segments, ng)
    blk_plan = None
    if args.workload == "muonbp":
        segs, ngb = H.blocked_segments(cfg["rows"], cfg["cols"], cfg["block_rows"], cfg["block_cols"])
        blk_plan = q.Plan(trip, segs, ngb)
    ws_u = plan.workspace()
    inv = torch.empty(ng, dtype=torch.float32, device=dev)
    hp = q.make_hparams(beta=H.BETA, eps=H.NS_EPS, coeffs=H.NS_COEFFS, lr_full=0.02, lr_block=0.01,
                        rms_scale=0.2, ns_steps=H.NS_STEPS,
                        period=cfg["period"] if args.workload == "muonbp" else 1)
    ws_ns = None
    if mats:
        nbytes = q.muon_step_workspace_bytes(plan, blk_plan, mats)
        ws_ns = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step(t, ev):
        if args.workload == "layerset28":
            ev[0].record()
            q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv, ws=ws_u)
            ev[1].record()
            ev[2].record()
        elif args.workload == "llama8b":
            ev[0].record()
            q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, False, group_inv_norm=inv, ws=ws_u)
            ev[1].record()
            q.muon_apply(plan, mats, True, inv, hp, ws_ns)
            ev[2].record()
        else:
            ev[0].record()
            q.muon_step(plan, blk_plan, mats, t, hp, ws=ws_ns)
            ev[1].record()
            ev[2].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for t in range(1, args.warmup + 1):
        step(t, mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for t in range(args.steps):
        step(args.warmup + 1 + t, evs[t])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    if args.ref_copy_mib > 0:
        src = torch.empty(args.ref_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    upd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ns_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_per_step = total_ms / args.steps

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic"}
    if args.workload == "layerset28":
        bytes_ = numel * (BYTES_PER_ELEM_UPDATE + BYTES_PER_ELEM_SCALE)
        gbs = bytes_ / (upd_ms * 1e-3) / 1e9
        out.update({"value": round(gbs, 2), "unit": "GB/s", "dtype": "f32",
                    "config": {"workload": "layerset28_grouped_update_normalize", "tensors": len(tensors),
                               "groups": ng, "elements": numel, "grad_dtype": "bf16", "state": "int8"},
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}})
    elif args.workload == "llama8b":
        bytes_ = numel * BYTES_PER_ELEM_UPDATE
        gbs = bytes_ / (upd_ms * 1e-3) / 1e9
        flops = sum(ns_sym_flops(r, c, H.NS_STEPS) for _, r, c in tensors)
        tfl = flops / (ns_ms * 1e-3) / 1e12
        out.update({"value": round(gbs, 2), "unit": "GB/s", "dtype": "bf16",
                    "ns_tflops": round(tfl, 2),
                    "config": {"workload": "llama8b_layer_muon_step", "matrices": len(tensors),
                               "elements": numel, "ns_steps": H.NS_STEPS, "ns_precision": "bf16",
                               "grad_dtype": "bf16", "state": "int8", "update_ms": round(upd_ms, 4),
                               "ns_apply_ms": round(ns_ms, 4), "ns_flops_per_step": flops},
                    "roofline": {"bound": "mfma", "achieved": round(tfl, 2), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                                 "traffic": None},
                    "roofline_update": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                        "traffic": None}})
    else:
        out.update({"value": round(1000.0 / ms_per_step, 3), "unit": "steps/s", "dtype": "bf16",
                    "config": {"workload": "muonbp_4096x14336_P5", "blocks": 8}})
    if host_q is not None:
        out["cpu_baseline"] = cpu_baseline(host_q, host_ns, H.NS_STEPS)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
