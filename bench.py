#!/usr/bin/env python3
"""Benchmark of one quantized-momentum Muon step on one MI355X.

Default workload: the Llama-8B-shaped layer (q/o 4096x4096, k/v 1024x4096,
gate/up 14336x4096, down 4096x14336), bf16 grads ~N(0, 1e-3), int8 momentum
state, one norm group per matrix; a step is the full Muon step: q8 update +
group norms (qmuon_update_normalize_groups), then quintic Newton-Schulz
(T = 5, bf16 MFMA) of every matrix with the weight update fused into its last
product (muon_apply).  muon_step is exactly these two calls; they are issued
separately here so HIP events on the launch stream time each phase live.

Printed: one JSON line.  value = q8 update GB/s over the whole update +
group-norm call (algorithmic bytes: int8 codes read+write, bf16 grad
read+write, fp32 absmax read+write per 256 elements = 6.03125 B/element);
ns_tflops = NS TFLOP/s over the whole muon_apply call (algorithmic FLOPs, the
two symmetric products at lower-triangle cost).  `roofline` is for the
dominant kernel (the one with the largest share of device time, measured live
per launch with the library's event timer over the timed steps: the
X <- aX + BX product, MFMA bound); `roofline_update` for the HBM-bound q8
update kernel.  The event timer runs on the even-numbered timed steps only:
its events cost the stream about 14 us per update call and 0.1 ms per step,
so value, ns_tflops and per_step_ms come from the odd-numbered steps, the
per-kernel figures from the even ones; ms_per_step is the whole timed region
over all steps.  `traffic` is filled from the committed counter summary only
while the kernel source still has the hash recorded there.  `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.

--carrier: the same step with m handed to Newton-Schulz as the MXFP8 carrier
(muon_step with hparams.carrier = 1: the update writes E4M3 bytes + per-32
E8M0 scales, 5.0625 B/element, and the NS prologue decodes them); the update
/ NS split then comes from the per-kernel timer.

The default run (llama8b without --carrier, --extras on) also measures the
three other full-size workloads, each in its own timed region after the
headline's buffers are freed, and adds them to the same JSON line:
  layerset28: the 28-layer 2048-hidden set, grouped update + normalisation
              (10.03 B/element), GB/s and fraction of HBM peak;
  muonbp:     4096x14336 in 8 column blocks, P = 5, steps 1..20: ms per step,
              NS TFLOP/s (symmetric FLOPs of all 20 steps over the NS-phase
              event time) and fraction of bf16 peak, the dominant kernel's
              live roofline;
  grasp:      GRASP 4096x4096 rank 8: steps/s, state-path GB/s, f32 NS
              TFLOP/s and fraction of the fp32 MFMA peak.

Other workloads (not the headline): --workload layerset28 (the 28-layer
2048-hidden set, grouped update + normalisation only), --workload muonbp
(4096x14336, 8 column blocks, P = 5), --workload grasp (GRASP 4096x4096,
rank 8: steps/s, state-path GB/s and f32 NS TFLOP/s against the fp32 peak),
--workload fp32_256x512 (one small fp32 matrix, latency in us per step),
--workload hbm_stream (the library's stream copy at the update's byte counts:
the achievable HBM rate of a 50/50 read/write stream).
per_step_ms gives the 10/50/90th percentiles of the per-step event times (odd-numbered steps).
"""
import argparse
import hashlib
import json
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
BYTES_PER_ELEM_SUMS = 3.015625       # 1 code, 2 bf16 grad, 4/256 absmax read (sums pass)
# The grouped update + normalisation is counted as the update followed by an
# in-place normalise pass, 10.03 B/element; the library moves 9.05 (a sums
# pass, then the update writing normalised values), so the call's GB/s on
# this basis is its speed against that two-kernel formulation.
NORMALIZE_BASIS = "10.03 B/element: update 6.03 + in-place normalise pass 4; moved: sums pass 3.02 + normalising update 6.03"
BYTES_PER_ELEM_CARRIER = 5.0625      # 1+1 code, 2 bf16 grad read, 1 + 1/32 carrier write, 8/256 absmax


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "layerset28", "muonbp", "grasp", "fp32_256x512", "hbm_stream"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: skip the layerset28 / muonbp / grasp sub-results")
    ap.add_argument("--rounding", default="nearest", choices=["nearest", "stochastic"],
                    help="requantisation rounding of the update (the headline uses nearest)")
    ap.add_argument("--carrier", action="store_true",
                    help="hand m to Newton-Schulz as the MXFP8 carrier (muon_step with hparams.carrier = 1) "
                         "instead of bf16 in the grads (llama8b and muonbp workloads)")
    ap.add_argument("--ns-precision", default="f32", choices=["f32", "bf16x3"],
                    help="fp32-operand NS arithmetic of the grasp and fp32_256x512 workloads: fp32 MFMAs, or "
                         "bf16 MFMAs on a hi + lo split of each operand")
    ap.add_argument("--ref-copy-mib", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB once (a kernel of "
                         "known traffic, to calibrate HBM byte counters in a profiler run)")
    return ap.parse_args()


def ns_sym_flops(rows, cols, steps):
    m, n = min(rows, cols), max(rows, cols)
    return steps * (n * m * (m + 1) + m * m * (m + 1) + 2 * m * m * n)


# Algorithmic work of one launch of each timed kernel class over a set of
# matrices (rows, cols): FLOPs for the products, bytes for memory kernels.
def launch_work(tensors, numel, carrier=False):
    mn = [(min(r, c), max(r, c)) for _, r, c in tensors]
    return {
        "ns_gram": ("mfma", sum(m * (m + 1) * n for m, n in mn)),
        "ns_poly": ("mfma", sum(m * m * (m + 1) for m, n in mn)),
        "ns_xupdate": ("mfma", sum(2 * m * m * n for m, n in mn)),
        "q8_update": ("hbm", numel * (BYTES_PER_ELEM_CARRIER if carrier else BYTES_PER_ELEM_UPDATE)),
        # bf16 m in (or the carrier: 1 + 1/32), bf16 X out
        "ns_prologue": ("hbm", numel * ((1 + 1 / 32) if carrier else 2.0) + numel * 2.0),
        "ns_writeback": ("hbm", numel * 12.0),   # bf16 X in, bf16 out, fp32 W read + write
    }


def source_hash(name):
    path = os.path.join(ROOT, "quantized_momentum_newton_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch from the committed counter summary, per kernel
    class, kept only while the kernel's source hash matches the one recorded."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return {}
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-json:"):
                rec = json.loads(line.split(":", 1)[1])
    if not rec:
        return {}
    out = {}
    for cls, v in rec.get("per_launch_bytes", {}).items():
        src = rec.get("sources", {}).get(cls)
        if src and source_hash(src["file"]) == src["sha256_16"]:
            out[cls] = v
    return out


def roofline(kind, work, ms_per_launch, traffic):
    if kind == "mfma":
        achieved = work / (ms_per_launch * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    achieved = work / (ms_per_launch * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}


def cpu_baseline(host_q, host_ns, steps):
    """The oracle as it stands, on a bounded sample of the same workload: the
    q8 update of every tensor of the layer (C oracle) and fp64 NS of the
    given matrices (numpy oracle)."""
    import oracle
    from oracle import ns
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count()
    numel = 0
    t0 = time.perf_counter()
    for codes, absmax, grad in host_q:
        oracle.q8_update(codes, absmax, grad, 0.95, oracle.BF16)
        numel += codes.size
    t_q = time.perf_counter() - t0
    gbs = numel * BYTES_PER_ELEM_UPDATE / t_q / 1e9
    fl, t_ns = 0, 0.0
    for x in host_ns:
        t0 = time.perf_counter()
        ns.ns_orthogonalize(x, steps)
        t_ns += time.perf_counter() - t0
        fl += ns_sym_flops(x.shape[0], x.shape[1], steps)
    shapes = " + ".join(f"{x.shape[0]}x{x.shape[1]}" for x in host_ns)
    return {
        "value": round(gbs, 3), "unit": "GB/s", "cores": max(oracle.num_threads(), blas_threads),
        "kind": "oracle",
        "sample": (f"q8 update of all {len(host_q)} tensors of the layer ({numel} bf16 elements, C oracle, once) + "
                   f"fp64 NS T={steps} of {shapes} (numpy oracle); NS TFLOP/s counts the symmetric FLOPs"),
        "ns_tflops": round(fl / t_ns / 1e12, 5),
        "q8_seconds": round(t_q, 3), "ns_seconds": round(t_ns, 3),
    }


def percentiles(ms):
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(p10), 4), "p50": round(float(p50), 4), "p90": round(float(p90), 4)}


def bench_grasp(args, q, H, torch):
    """GRASP 4096x4096 (rank 8): one grasp_step per step on a fresh bf16 grad
    (noise + a fixed rank-8 spike); the state path and the fp32-operand NS
    (T = 5) in the arithmetic --ns-precision names."""
    cfg = H.grasp_4096_shape()
    rows, cols, k = cfg["rows"], cfg["cols"], cfg["rank"]
    dev = "cuda"
    spike = H.spike(rows, cols, k, dev, 1005)
    warm = H.gaussian((cols, k), dev, 1005)
    grads = [(H.grad((rows, cols), torch.float32, dev, 1005, t) + spike).to(torch.bfloat16) for t in range(4)]
    st = q.GraspState(rows, cols, k)
    ws = torch.empty(q.grasp_workspace_bytes(rows, cols, k), dtype=torch.uint8, device=dev)
    g = torch.empty_like(grads[0])
    def step(i, e):
        g.copy_(grads[(i - 1) % 4])
        e[0].record()
        q.grasp_step(st, g, warm, mu=cfg["mu"], ns_steps=H.NS_STEPS, coeffs=H.NS_COEFFS, eps=H.NS_EPS, ws=ws,
                     ns_precision=args.ns_precision)
        e[1].record()

    evs, pc, _ = timed_steps(args, torch, q, step, 2)
    ms = [evs[k][0].elapsed_time(evs[k][1]) for k in call_steps(args.steps)]
    step_ms = sum(ms) / len(ms)
    ns_ms = sum(pc[c][0] for c in ("ns_norm", "ns_prologue", "ns_gram", "ns_poly", "ns_xupdate",
                                   "ns_writeback")) / len(timer_steps(args.steps))
    state_ms = step_ms - ns_ms
    numel = rows * cols
    state_bytes = numel * 15.25             # three passes over the fp32 momentum plus the codes
    ns_fl = ns_sym_flops(rows, cols, H.NS_STEPS)
    # the arithmetic's own ceiling: the fp32 MFMA peak, or a third of the
    # bf16 MFMA peak for bf16x3 (three bf16 products per fp32 product)
    peak = F32_PEAK_TFLOPS if args.ns_precision == "f32" else BF16_PEAK_TFLOPS / 3
    return {"metric": METRIC, "value": round(1000.0 / step_ms, 3), "unit": "steps/s", "dtype": args.ns_precision,
            "ms_per_step": round(step_ms, 4), "per_step_ms": percentiles(ms),
            "config": {"workload": "grasp_4096x4096_rank8", "ns_steps": H.NS_STEPS, "ns_precision": args.ns_precision,
                       "state_ms": round(state_ms, 4), "ns_ms": round(ns_ms, 4),
                       "state_gbs": round(state_bytes / (state_ms * 1e-3) / 1e9, 1),
                       "ns_tflops": round(ns_fl / (ns_ms * 1e-3) / 1e12, 2),
                       "ns_peak_tflops": round(peak, 1),
                       "ns_frac_of_peak": round(ns_fl / (ns_ms * 1e-3) / 1e12 / peak, 4)}}


def bench_small(args, q, H, torch):
    """One 256x512 fp32 matrix: update + normalise + f32 NS (T = 5) + weight
    apply through muon_step.  Latency-bound (1.3 MB, 0.6 GFLOP): reported as
    microseconds per step."""
    (_, r, c), = H.fp32_256x512_shapes()
    dev = "cuda"
    codes, absmax = H.prior_state(r * c, dev, 1001, 0)
    g0 = H.grad((r, c), torch.float32, dev, 1001, 0).reshape(-1)
    g = g0.clone()
    w = H.weights((r, c), dev, 1001, 0)
    plan = q.Plan([(codes, absmax, g)], [(0, 0, r * c, 0)], 1)
    mats = [(r, c, r, c, w)]
    hp = q.make_hparams(beta=H.BETA, eps=H.NS_EPS, coeffs=H.NS_COEFFS, ns_steps=H.NS_STEPS, period=1,
                        precision=args.ns_precision)
    ws = torch.empty(q.muon_step_workspace_bytes(plan, None, mats, hparams=hp), dtype=torch.uint8, device=dev)
    evs = []
    for t in range(args.warmup + args.steps):
        g.copy_(g0)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        q.muon_step(plan, None, mats, t + 1, hp, ws=ws)
        e[1].record()
        if t >= args.warmup:
            evs.append(e)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    step_ms = sum(ms) / len(ms)
    return {"metric": METRIC, "value": round(step_ms * 1e3, 2), "unit": "us/step", "dtype": args.ns_precision,
            "higher_is_better": False, "ms_per_step": round(step_ms, 4), "per_step_ms": percentiles(ms),
            "config": {"workload": "fp32_256x512_muon_step", "ns_steps": H.NS_STEPS,
                       "ns_precision": args.ns_precision}}


def bench_hbm_stream(args, q, H, torch):
    """The achievable HBM rate for a 50/50 read/write stream: the library's
    stream copy (the q8 update's access pattern) over as many bytes as the
    q8 update moves on the Llama-8B layer (read + write = 6.03125 B/element x
    218M elements) and on the 28-layer set (x 1.32G elements)."""
    out = {}
    for name, numel in (("llama8b_layer_update_bytes", 218103808), ("layerset28_update_bytes", 1321205760)):
        n = int(numel * BYTES_PER_ELEM_UPDATE / 2) // 4096 * 4096      # bytes read = bytes written
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        evs = []
        for t in range(args.warmup + args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            q.hbm_stream_copy(src, dst)
            e[1].record()
            if t >= args.warmup:
                evs.append(e)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
        avg = sum(ms) / len(ms)
        out[name] = {"bytes_per_copy": 2 * n, "ms": round(avg, 4), "gbs": round(2 * n / (avg * 1e-3) / 1e9, 1),
                     "per_copy_ms": percentiles(ms)}
        del src, dst
        torch.cuda.empty_cache()
    head = out["llama8b_layer_update_bytes"]
    return {"metric": METRIC, "value": head["gbs"], "unit": "GB/s", "dtype": "u8",
            "ms_per_step": head["ms"], "frac": round(head["gbs"] / HBM_PEAK_GBS, 4),
            "config": {"workload": "hbm_stream_copy", "sizes": out}}


def timer_steps(n):
    """Timed steps that run the library's per-kernel timer: the even-numbered
    ones.  Its events ride on the dispatches but still cost the stream a few
    microseconds per launch group (about 14 us on the headline update call),
    so whole-call figures come from the other steps (all of them when fewer
    than two are timed)."""
    return [k for k in range(n) if k % 2 == 0]


def call_steps(n):
    return [k for k in range(n) if k % 2 == 1] if n >= 2 else list(range(n))


def timed_steps(args, torch, q, step, n_events):
    """Warm-up steps, then args.steps timed steps with n_events HIP events per
    step (recorded on torch's current stream, which the library launches on),
    the library's per-kernel timer on the steps timer_steps names.
    step(i, events): i counts from 1 over warm-up and timed steps.  Returns
    (per-step event lists, per-class (ms, launches) over the timer steps,
    total ms)."""
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    for i in range(1, args.warmup + 1):
        step(i, mk())
    evs = [mk() for _ in range(args.steps)]
    timed = set(timer_steps(args.steps))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        if k in timed:
            q.timing_enable(True, resume=k > 0)
        step(args.warmup + 1 + k, evs[k])
        if k in timed:
            q.timing_enable(False)
    stop.record()
    torch.cuda.synchronize()
    return evs, {k: q.timing_read(k) for k in q.KERNEL_CLASSES}, start.elapsed_time(stop)


def extra_layerset28(args, q, H, torch):
    """28-layer set: one grouped update + normalisation per step (write-back of
    the normalised grads), 10.03 B/element."""
    tensors, segments, ng = H.layerset28_layout()
    trip, numel = [], 0
    for i, (_, r, c) in enumerate(tensors):
        codes, absmax = H.prior_state(r * c, "cuda", 1002, i)
        g = H.grad((r, c), torch.bfloat16, "cuda", 1002, i, outlier_frac=0.01).reshape(-1)
        trip.append((codes, absmax, g))
        numel += r * c
    plan = q.Plan(trip, segments, ng)
    ws = plan.workspace()
    inv = torch.empty(ng, dtype=torch.float32, device="cuda")

    def step(i, ev):
        ev[0].record()
        q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv, ws=ws)
        ev[1].record()

    evs, pc, total = timed_steps(args, torch, q, step, 2)
    cs = call_steps(args.steps)
    ms = sum(evs[k][0].elapsed_time(evs[k][1]) for k in cs) / len(cs)
    gbs = numel * (BYTES_PER_ELEM_UPDATE + BYTES_PER_ELEM_SCALE) / (ms * 1e-3) / 1e9
    moved = numel * (BYTES_PER_ELEM_UPDATE + BYTES_PER_ELEM_SUMS) / (ms * 1e-3) / 1e9
    upd_ms, n = pc["q8_update"]
    rl = roofline("hbm", numel * BYTES_PER_ELEM_UPDATE, upd_ms / n, None)
    rl["kernel"] = "q8_update"
    return {"value": round(gbs, 2), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_per_step": round(ms, 4),
            "moved_gbs": round(moved, 2), "moved_frac": round(moved / HBM_PEAK_GBS, 4),
            "config": {"workload": "layerset28_grouped_update_normalize", "tensors": len(tensors), "groups": ng,
                       "elements": numel, "grad_dtype": "bf16", "state": "int8", "bytes_basis": NORMALIZE_BASIS},
            "roofline": rl,
            "kernels": {k: round(v[0] / v[1], 4) for k, v in pc.items() if v[1]}}


def extra_muonbp(args, q, H, torch):
    """MuonBP 4096x14336, 8 column blocks of 4096x1792, P = 5: the update with
    the step's plan, then NS + weight apply (muon_step's two halves, so events
    time the NS phase).  Timed steps are numbered 1.. after the warm-up, so a
    20-step region holds 16 block steps and 4 full steps."""
    cfg = H.muonbp_4096x14336_shape()
    r, c, br, bc = cfg["rows"], cfg["cols"], cfg["block_rows"], cfg["block_cols"]
    codes, absmax = H.prior_state(r * c, "cuda", 1004, 0)
    g = H.grad((r, c), torch.bfloat16, "cuda", 1004, 0).reshape(-1)
    w = H.weights((r, c), "cuda", 1004, 0)
    trip, mats = [(codes, absmax, g)], [(r, c, br, bc, w)]
    full = q.Plan(trip, [(0, 0, r * c, 0)], 1)
    segs, ngb = H.blocked_segments(r, c, br, bc)
    blk = q.Plan(trip, segs, ngb)
    hp = q.make_hparams(beta=H.BETA, eps=H.NS_EPS, coeffs=H.NS_COEFFS, lr_full=cfg["lr_full"],
                        lr_block=cfg["lr_block"], rms_scale=cfg["rms_scale"], ns_steps=H.NS_STEPS,
                        period=cfg["period"])
    ws = torch.empty(q.muon_step_workspace_bytes(full, blk, mats, hparams=hp), dtype=torch.uint8, device="cuda")
    ws_u = torch.empty(max(full.workspace_bytes(), blk.workspace_bytes()), dtype=torch.uint8, device="cuda")
    inv = {True: torch.empty(1, dtype=torch.float32, device="cuda"),
           False: torch.empty(ngb, dtype=torch.float32, device="cuda")}
    period = cfg["period"]
    kinds = []

    def step(i, ev):
        t = i if i <= args.warmup else i - args.warmup      # timed steps restart at t = 1
        is_full = t % period == 0
        p = full if is_full else blk
        ev[0].record()
        q.qmuon_update_normalize_groups(p, H.BETA, H.NS_EPS, False, group_inv_norm=inv[is_full], ws=ws_u)
        ev[1].record()
        q.muon_apply(p, mats, is_full, inv[is_full], hp, ws)
        ev[2].record()
        if i > args.warmup:
            kinds.append(is_full)

    evs, pc, total = timed_steps(args, torch, q, step, 3)
    cs = call_steps(args.steps)
    ns_ms = sum(evs[k][1].elapsed_time(evs[k][2]) for k in cs)
    step_ms = [evs[k][0].elapsed_time(evs[k][2]) for k in cs]
    m_b, n_b = min(br, bc), max(br, bc)
    m_f, n_f = min(r, c), max(r, c)
    nblk = (r // br) * (c // bc)
    fl = sum(ns_sym_flops(r, c, H.NS_STEPS) if kinds[k] else nblk * ns_sym_flops(br, bc, H.NS_STEPS) for k in cs)
    # algorithmic work of every launch of each product class over the timer steps
    tk = [kinds[k] for k in timer_steps(args.steps)]
    n_full = sum(tk)
    n_blk = len(tk) - n_full
    T = H.NS_STEPS
    work = {"ns_gram": T * (n_full * m_f * (m_f + 1) * n_f + n_blk * nblk * m_b * (m_b + 1) * n_b),
            "ns_poly": T * (n_full * m_f * m_f * (m_f + 1) + n_blk * nblk * m_b * m_b * (m_b + 1)),
            "ns_xupdate": T * (n_full * 2 * m_f * m_f * n_f + n_blk * nblk * 2 * m_b * m_b * n_b)}
    dom = max(work, key=lambda k: pc[k][0])
    rl = roofline("mfma", work[dom], pc[dom][0], None)   # all launches: total work over total time
    rl["kernel"] = dom
    tfl = fl / (ns_ms * 1e-3) / 1e12
    return {"value": round(1000.0 * len(step_ms) / sum(step_ms), 3), "unit": "steps/s",
            "ms_per_step": round(sum(step_ms) / len(step_ms), 4), "per_step_ms": percentiles(step_ms),
            "ns_tflops": round(tfl, 2), "ns_frac": round(tfl / BF16_PEAK_TFLOPS, 4),
            "ns_ms_total": round(ns_ms, 3), "ns_flops_total": fl,
            "full_steps": sum(kinds[k] for k in cs), "block_steps": sum(not kinds[k] for k in cs),
            "config": {"workload": "muonbp_4096x14336_P5", "blocks": nblk, "block_shape": [br, bc],
                       "ns_steps": T, "ns_precision": "bf16"},
            "roofline": rl,
            "kernels": {k: {"ms": round(v[0], 3), "launches": v[1]} for k, v in pc.items() if v[1]}}


def extra_grasp(args, q, H, torch):
    """GRASP 4096x4096 rank 8 with the fp32-MFMA NS (the bench_grasp line)."""
    a = argparse.Namespace(**vars(args))
    a.ns_precision = "f32"
    r = bench_grasp(a, q, H, torch)
    cfg = r["config"]
    return {"value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
            "per_step_ms": r["per_step_ms"], "state_gbs": cfg["state_gbs"], "ns_tflops": cfg["ns_tflops"],
            "ns_frac_of_f32_peak": cfg["ns_frac_of_peak"], "ns_peak_tflops": cfg["ns_peak_tflops"],
            "config": {"workload": cfg["workload"], "ns_steps": cfg["ns_steps"], "ns_precision": "f32"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_momentum_newton_amd as q
    from harness import inputs as H
    torch.cuda.init()
    if args.workload in ("grasp", "fp32_256x512", "hbm_stream"):
        fn = {"grasp": bench_grasp, "fp32_256x512": bench_small, "hbm_stream": bench_hbm_stream}[args.workload]
        out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
        out.update(fn(args, q, H, torch))
        print(json.dumps(out), flush=True)
        return
    out = bench_layer(args, q, H, torch)
    if args.workload == "llama8b" and not args.carrier and not args.no_extras:
        # the three other full-size workloads, each in its own timed region
        for name, fn in (("layerset28", extra_layerset28), ("muonbp", extra_muonbp), ("grasp", extra_grasp)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            out[name] = fn(args, q, H, torch)
    print(json.dumps(out), flush=True)


def bench_layer(args, q, H, torch):
    """The llama8b / layerset28 / muonbp workloads as the headline line."""
    dev = "cuda"

    if args.workload == "llama8b":
        tensors, segments, ng = H.llama8b_layer_layout()
    elif args.workload == "layerset28":
        tensors, segments, ng = H.layerset28_layout()
    else:
        cfg = H.muonbp_4096x14336_shape()
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
    if not args.no_cpu_baseline and args.workload == "llama8b":
        import numpy as np
        host_q = [(c.cpu().numpy(), a.cpu().numpy(), g.view(torch.int16).cpu().numpy().view(np.uint16))
                  for c, a, g in trip]
        # NS sample: the q (4096 x 4096), k (1024 x 4096), gate (14336 x 4096)
        # and down (4096 x 14336) matrices, about 10 s of fp64 work on 16 host cores
        pick = [next(i for i, t in enumerate(tensors) if t[0] == nm) for nm in ("q", "k", "gate", "down")]
        host_ns = [trip[i][2].float().cpu().numpy().astype(np.float64).reshape(tensors[i][1], tensors[i][2])
                   for i in pick]

    plan = q.Plan(trip, segments, ng)
    blk_plan = None
    if args.workload == "muonbp":
        segs, ngb = H.blocked_segments(cfg["rows"], cfg["cols"], cfg["block_rows"], cfg["block_cols"])
        blk_plan = q.Plan(trip, segs, ngb)
    ws_u = plan.workspace()
    inv = torch.empty(ng, dtype=torch.float32, device=dev)
    if args.carrier and (args.workload == "layerset28" or args.rounding != "nearest"):
        print("--carrier needs the llama8b or muonbp workload and nearest rounding", file=sys.stderr)
        sys.exit(2)
    hp = q.make_hparams(beta=H.BETA, eps=H.NS_EPS, coeffs=H.NS_COEFFS, lr_full=0.02, lr_block=0.01,
                        rms_scale=0.2, ns_steps=H.NS_STEPS,
                        period=cfg["period"] if args.workload == "muonbp" else 1, carrier=args.carrier)
    ws_ns = None
    if mats:
        nbytes = q.muon_step_workspace_bytes(plan, blk_plan, mats, hparams=hp)
        ws_ns = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step(t, ev):
        if args.workload == "layerset28":
            ev[0].record()
            q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, True, group_inv_norm=inv, ws=ws_u,
                                            rounding=args.rounding, seed=1234, offset=t)
            ev[1].record()
            ev[2].record()
        elif args.workload == "llama8b" and args.carrier:
            # one call; the update / NS split comes from the per-kernel timer
            ev[0].record()
            q.muon_step(plan, None, mats, t, hp, ws=ws_ns)
            ev[1].record()
            ev[2].record()
        elif args.workload == "llama8b":
            ev[0].record()
            q.qmuon_update_normalize_groups(plan, H.BETA, H.NS_EPS, False, group_inv_norm=inv, ws=ws_u,
                                            rounding=args.rounding, seed=1234, offset=t)
            ev[1].record()
            q.muon_apply(plan, mats, True, inv, hp, ws_ns)
            ev[2].record()
        else:
            ev[0].record()
            q.muon_step(plan, blk_plan, mats, t, hp, ws=ws_ns)
            ev[1].record()
            ev[2].record()

    evs, per_class, total_ms = timed_steps(args, torch, q, step, 3)
    cs = call_steps(args.steps)
    n_timer = len(timer_steps(args.steps))
    if args.ref_copy_mib > 0:
        src = torch.empty(args.ref_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    upd_ms = sum(evs[k][0].elapsed_time(evs[k][1]) for k in cs) / len(cs)
    ns_ms = sum(evs[k][1].elapsed_time(evs[k][2]) for k in cs) / len(cs)
    if args.carrier and args.workload == "llama8b":
        call_ms = upd_ms
        upd_ms = (per_class["q8_update"][0] + per_class["group_reduce"][0]) / n_timer
        ns_ms = call_ms - upd_ms
    ms_per_step = total_ms / args.steps
    step_ms = [evs[k][0].elapsed_time(evs[k][2]) for k in cs]

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 4), "per_step_ms": percentiles(step_ms), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    if args.workload == "layerset28":
        bytes_ = numel * (BYTES_PER_ELEM_UPDATE + BYTES_PER_ELEM_SCALE)
        gbs = bytes_ / (upd_ms * 1e-3) / 1e9
        moved = numel * (BYTES_PER_ELEM_UPDATE + BYTES_PER_ELEM_SUMS) / (upd_ms * 1e-3) / 1e9
        per_elem = {"q8_update": BYTES_PER_ELEM_UPDATE, "q8_scale": BYTES_PER_ELEM_SCALE, "q8_sums": BYTES_PER_ELEM_SUMS}
        kernels = {k: {"ms_per_launch": round(ms / n, 4), "launches": n,
                       "gbs": round(numel * per_elem.get(k, 0.0) / (ms / n * 1e-3) / 1e9, 1)}
                   for k, (ms, n) in per_class.items() if n}
        ms_u, n_u = per_class["q8_update"]
        rl = roofline("hbm", numel * BYTES_PER_ELEM_UPDATE, ms_u / n_u, None)
        rl["kernel"] = "q8_update"
        out.update({"value": round(gbs, 2), "unit": "GB/s", "dtype": "bf16",
                    "moved_gbs": round(moved, 2), "moved_frac": round(moved / HBM_PEAK_GBS, 4),
                    "config": {"workload": "layerset28_grouped_update_normalize", "tensors": len(tensors),
                               "groups": ng, "elements": numel, "grad_dtype": "bf16", "state": "int8",
                               "bytes_basis": NORMALIZE_BASIS},
                    "roofline": rl,
                    "kernels": kernels})
    elif args.workload == "llama8b":
        bytes_ = numel * (BYTES_PER_ELEM_CARRIER if args.carrier else BYTES_PER_ELEM_UPDATE)
        gbs = bytes_ / (upd_ms * 1e-3) / 1e9
        flops = sum(ns_sym_flops(r, c, H.NS_STEPS) for _, r, c in tensors)
        tfl = flops / (ns_ms * 1e-3) / 1e12
        work = launch_work(tensors, numel, args.carrier)
        traffic = recorded_traffic("llama8b_layer_carrier" if args.carrier else "llama8b_layer")
        kernels = {k: {"ms_per_launch": round(ms / n, 4), "launches": n, "share": round(ms / total_ms, 4)}
                   for k, (ms, n) in per_class.items() if n}
        timed = [k for k in work if per_class[k][1]]
        dom = max(timed, key=lambda k: per_class[k][0])
        rl = {}
        for k in (dom, "q8_update"):
            ms, n = per_class[k]
            rl[k] = roofline(work[k][0], work[k][1], ms / n, traffic.get(k))
            rl[k]["kernel"] = k
        out.update({"value": round(gbs, 2), "unit": "GB/s", "dtype": "bf16",
                    "ns_tflops": round(tfl, 2),
                    "config": {"workload": "llama8b_layer_muon_step", "matrices": len(tensors),
                               "elements": numel, "ns_steps": H.NS_STEPS, "ns_precision": "bf16",
                               "grad_dtype": "bf16", "state": "int8", "rounding": args.rounding,
                               "handoff": "mxfp8_carrier" if args.carrier else "bf16_grad",
                               "update_ms": round(upd_ms, 4),
                               "ns_apply_ms": round(ns_ms, 4), "ns_flops_per_step": flops},
                    "roofline": rl[dom], "roofline_update": rl["q8_update"], "kernels": kernels})
    else:
        out.update({"value": round(1000.0 / ms_per_step, 3), "unit": "steps/s", "dtype": "bf16",
                    "config": {"workload": "muonbp_4096x14336_P5", "blocks": 8,
                               "handoff": "mxfp8_carrier" if args.carrier else "bf16_grad"}})
    if host_q is not None:
        out["cpu_baseline"] = cpu_baseline(host_q, host_ns, H.NS_STEPS)
    return out


if __name__ == "__main__":
    main()
