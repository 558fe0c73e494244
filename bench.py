#!/usr/bin/env python3
"""Benchmark of the PAB attention hot path on one MI355X.

One benchmark step is one whole denoising trajectory of the 480p-latent DiT
block (48 frames x 1590 tokens, 16 heads x 72, 120 text tokens, 30 steps,
broadcast ranges spatial 2 / temporal 4 / cross 6, bf16): the schedule from
pab_plan_schedule, then per step pab_step_dispatch for each attention type
(spatial, temporal and cross kernels on recompute steps, nothing on
broadcast steps), each recompute also taking the attention-difference MSE
against the previous computation of its type (the quantity the pages plot to
motivate the broadcast ranges, used to calibrate them; the dispatcher folds
it into the attention kernels' output pass).  All inputs of the trajectory
are generated into HBM before timing starts.  The same trajectory without
the difference, as a production run would take it, is reported beside it.

Prints one JSON line: metric, value (attention TFLOP/s executed per second
of PAB-on trajectory), ms_per_step (ms per PAB-on trajectory), the PAB-off
trajectory beside it, per-kernel timings, the roofline of the dominant
kernel (spatial attention, bf16 MFMA) measured live with HIP events on the
launch stream, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config b480|b720|full3d|cfg480|stack28|tiny]
                    [--module-config b480m|""] [--stream-inputs] [--no-peaks]
                    [--no-cpu-baseline] [--calib-copy]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and ms per denoise trajectory (PAB on/off), % of roofline"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_b480.md")
KERNEL_SOURCES = {
    "spatial": "reuse_pab_plan_amd/csrc/spatial.hip",
    "temporal": "reuse_pab_plan_amd/csrc/temporal.hip",
    "cross": "reuse_pab_plan_amd/csrc/cross.hip",
    "mse": "reuse_pab_plan_amd/csrc/mse.hip",
}


def source_hash(rel):
    with open(os.path.join(ROOT, rel), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_traffic(config, kernel):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    tr = json.loads(text[start + 7:end])
    k = tr.get("kernels", {}).get(kernel)
    if tr.get("config") != config or not k or k.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return k.get("hbm_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed PAB-on trajectories")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--off-steps", type=int, default=5, help="timed PAB-off trajectories")
    ap.add_argument("--config", default="b480")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--module-config", default="b480m",
                    help="attention-module workload timed after the main line ('' to skip)")
    ap.add_argument("--module-steps", type=int, default=3)
    ap.add_argument("--stream-inputs", action="store_true",
                    help="generate each step's inputs between dispatches instead of keeping all "
                         "of them resident (workloads too large for HBM, e.g. stack28); times are "
                         "then the sum of the kernel brackets, not the trajectory wall time")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the sustained-peak microbenchmarks (measured roofline denominators)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def stats_ms(pairs):
    import numpy as np

    ms = np.array([a.elapsed_time(b) for a, b in pairs], dtype=np.float64)
    if ms.size == 0:
        return None
    return {"n": int(ms.size), "mean_ms": float(ms.mean()), "median_ms": float(np.median(ms)),
            "p10_ms": float(np.percentile(ms, 10)), "p90_ms": float(np.percentile(ms, 90))}


def cpu_baseline(cfg, traj_on, inputs, budget_s):
    """Time the oracle (as it stands) on a bounded sample of the same workload.

    Per attention type: oracle outputs for whole (b, h) slices of one
    recompute step's inputs, adding heads until the type's share of the time
    budget is used, and one oracle MSE call.  The oracle's trajectory time is
    derived as sum_a count_a * flops_a / rate_a (every call of a type has the
    same shape) plus one MSE per recompute that has a predecessor.
    """
    import numpy as np
    import threadpoolctl

    import oracle
    from reuse_pab_plan_amd import harness

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    per_type = budget_s / len(cfg.kinds)
    rates, sample = [], []
    step = 0
    for a, kind in enumerate(cfg.kinds):
        q, k, v = inputs.get(0, a, step)
        done_flops, t_used, heads = 0, 0.0, 0
        for b in range(cfg.B):
            for h in range(cfg.H):
                qh = q[b:b + 1, h:h + 1].float().cpu().numpy()
                kh = k[b:b + 1, h:h + 1].float().cpu().numpy()
                vh = v[b:b + 1, h:h + 1].float().cpu().numpy()
                t0 = time.perf_counter()
                if kind == "spatial":
                    oracle.spatial(qh, kh, vh)
                elif kind == "temporal":
                    oracle.temporal(qh, kh, vh)
                else:
                    oracle.cross(qh, kh, vh)
                t_used += time.perf_counter() - t0
                heads += 1
                done_flops += harness.attn_flops(cfg, kind) // (cfg.B * cfg.H)
                if t_used >= per_type:
                    break
            if t_used >= per_type:
                break
        rates.append(done_flops / t_used)
        sample.append(f"{kind}: {heads} of {cfg.B * cfg.H} (b,h) slices of one step")
    # The attention-difference MSE after each recompute that has a
    # predecessor (part of the timed step): the oracle MSE on two outputs.
    q0, k0, _ = inputs.get(0, 0, step)  # two tensors of the output's size
    o1, o2 = q0.float().cpu().numpy(), k0.float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.mse(o1, o2)
    mse_s = time.perf_counter() - t0
    n_mse = sum(max(int(traj_on.counts[a]) - 1, 0) for a in range(len(cfg.kinds))) * cfg.blocks
    sample.append(f"mse: one call on two video-sized tensors ({mse_s * 1e3:.0f} ms)")
    traj_s = sum(int(traj_on.counts[a]) * harness.attn_flops(cfg, kind) * cfg.blocks / rates[a]
                 for a, kind in enumerate(cfg.kinds)) + n_mse * mse_s
    value = traj_on.flops() / traj_s / 1e12
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "; ".join(sample) + f"; fp64 numpy oracle; trajectory time derived as "
                  f"sum of count x per-call time = {traj_s:.1f} s per PAB-on trajectory",
        "ms_per_trajectory": traj_s * 1e3,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def module_leg(name, steps, dev, stream):
    """Attention modules (input projection, attention, output projection
    around each attention type) over a PAB-on and a PAB-off trajectory, and
    the two projection GEMMs timed alone at the workload's shapes."""
    import numpy as np
    import torch

    from reuse_pab_plan_amd import harness, lib

    cfg = harness.CONFIGS[name]
    on = harness.Trajectory(cfg, pab=True, device=dev, stream=stream, drift=False)
    off = harness.Trajectory(cfg, pab=False, device=dev, stream=stream, drift=False)
    inputs = harness.Inputs(cfg, off.steps_needed(), device=dev, resident=True)
    on.inputs = off.inputs = inputs
    on.run(events=False)
    off.run(events=False)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for label, traj, n in (("on", on, steps), ("off", off, 1)):
        per = [[] for _ in cfg.kinds]
        start.record(stream)
        for _ in range(n):
            r = traj.run(events=True)
            for a in range(len(cfg.kinds)):
                per[a] += r["brackets"]["attn"][a]
        stop.record(stream)
        torch.cuda.synchronize()
        res[label] = (start.elapsed_time(stop) / n, per)
    on_ms, per_on = res["on"]
    off_ms, _ = res["off"]
    out = {"workload": cfg.desc, "name": cfg.name,
           "pab_on_ms_per_trajectory": on_ms, "pab_off_ms_per_trajectory": off_ms,
           "pab_speedup": off_ms / on_ms,
           "tflops_pab_on": on.flops() / (on_ms * 1e-3) / 1e12,
           "module_ms": {k: stats_ms(per_on[a])["mean_ms"] for a, k in enumerate(cfg.kinds)}}
    # The GEMMs alone, on the stream they are launched on, rotating over
    # three input sets so the timed launches read HBM.
    B, H, F, S, D = cfg.video_shape
    C_, T = cfg.C, F * S
    xs = [inputs.get(0, 0, i)[0] for i in range(3)]
    w_in, _, w_out = inputs.weights(0, 0)
    bufs = [[torch.empty(cfg.video_shape, dtype=torch.bfloat16, device=dev) for _ in range(3)]
            for _ in range(3)]
    ys = [torch.empty((B, T, C_), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    st = stream.cuda_stream
    gemms = {
        "proj_in": (lambda i: lib.pab_proj_in(xs[i % 3], w_in, bufs[i % 3], F, S, H, D, stream=st),
                    2 * B * T * 3 * C_ * C_),
        "proj_out": (lambda i: lib.pab_proj_out(bufs[i % 3][0], w_out, ys[i % 3], stream=st),
                     2 * B * T * C_ * C_),
    }
    out["gemm"] = {}
    for g, (fn, flops) in gemms.items():
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        ev = []
        for i in range(12):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(i)
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        sm = stats_ms(ev)
        sm["flops_per_launch"] = flops
        sm["tflops"] = flops / (sm["mean_ms"] * 1e-3) / 1e12
        sm["frac_mfma"] = sm["tflops"] / PEAK_BF16_TFLOPS
        out["gemm"][g] = sm
    del on, off, inputs, bufs, ys
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this PAB hot path has no multi-GPU mode "
              "(sequence-parallel sharding is a design note, not built). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from reuse_pab_plan_amd import harness, lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib.load()
    cfg = harness.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)

    traj_on = harness.Trajectory(cfg, pab=True, device=dev, stream=stream, drift=False)
    traj_off = harness.Trajectory(cfg, pab=False, device=dev, stream=stream, drift=False)
    t0 = time.time()
    # PAB-off needs every step's inputs; PAB-on uses a subset of them.
    needed = traj_off.steps_needed() if args.off_steps > 0 else traj_on.steps_needed()
    streamed = args.stream_inputs
    inputs = harness.Inputs(cfg, [] if streamed else needed, device=dev, resident=not streamed)
    traj_on.inputs = inputs
    traj_off.inputs = inputs
    torch.cuda.synchronize()
    log(f"config {cfg.name}: inputs generated in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB resident)")

    if args.calib_copy:
        # Plain copy of exactly 2 GiB read + 2 GiB written, for scaling the
        # FETCH_SIZE / WRITE_SIZE counters of the attention kernels.
        src = torch.empty(2**30, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # One bench step is one pass of the whole path: plan the schedule, then
    # the PAB-on trajectory -- each step's dispatch (attention kernels on
    # recompute steps, the cache slot in place on broadcast steps) and, after
    # each recompute, the attention-difference MSE against the previous
    # computation of its type (Figure 1's quantity).
    traj_on.drift = True
    for w in range(args.warmup):
        traj_on.replan()
        traj_on.run(events=False)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    brackets = {"attn": [[] for _ in cfg.kinds], "diff": [[] for _ in cfg.kinds]}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        traj_on.replan()
        r = traj_on.run(events=True)
        for a in range(len(cfg.kinds)):
            brackets["attn"][a] += r["brackets"]["attn"][a]
            brackets["diff"][a] += r["brackets"]["diff"][a]
    stop.record(stream)
    torch.cuda.synchronize()
    on_ms = start.elapsed_time(stop) / args.steps
    if streamed:  # kernel time only: inputs were generated between the dispatches
        on_ms = sum(a.elapsed_time(b) for v in brackets["attn"] for a, b in v) / args.steps
    log(f"PAB on (schedule, dispatch, attention-difference MSE): {on_ms:.3f} ms per trajectory")

    # The same trajectory as a production run would take it: no MSE.
    traj_on.drift = False
    n_prod = max(1, min(args.steps, 5))
    prod_kernel_ms = 0.0
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(n_prod):
        r_prod = traj_on.run(events=streamed)
        if streamed:
            torch.cuda.synchronize()
            prod_kernel_ms += sum(a.elapsed_time(b) for v in r_prod["brackets"]["attn"]
                                  for a, b in v)
    stop.record(stream)
    torch.cuda.synchronize()
    prod_ms = (prod_kernel_ms if streamed else start.elapsed_time(stop)) / n_prod
    log(f"PAB on without the MSE: {prod_ms:.3f} ms per trajectory")

    # Dispatch-mask check against the plan (bit-exact schedule in the timed runs).
    for a in range(len(cfg.kinds)):
        got = (r["masks"][0] >> a) & 1
        if not (got == traj_on.recompute[:, a]).all():
            raise RuntimeError(f"dispatch mask of type {a} differs from the schedule")

    off_ms = None
    calibration = None
    if args.off_steps > 0:
        # PAB off, the same pass (schedule, every step computed, MSE).
        traj_off.drift = True
        traj_off.run(events=False)
        torch.cuda.synchronize()
        start.record(stream)
        off_kernel_ms = 0.0
        for s in range(args.off_steps):
            traj_off.replan()
            r_off = traj_off.run(events=streamed)
            if streamed:
                torch.cuda.synchronize()
                off_kernel_ms += sum(a.elapsed_time(b) for v in r_off["brackets"]["attn"]
                                     for a, b in v)
        stop.record(stream)
        torch.cuda.synchronize()
        traj_off.drift = False
        off_ms = start.elapsed_time(stop) / args.off_steps
        if streamed:
            off_ms = off_kernel_ms / args.off_steps
        log(f"PAB off (schedule, dispatch, MSE): {off_ms:.3f} ms per trajectory")
        if not streamed:
            # Range calibration from the PAB-off trajectory's attention difference.
            t_cal = time.time()
            cal_ranges, cal_scores, _ = harness.calibrate(traj_off)
            calibration = {
                "candidates": list(cfg.ranges),
                "ranges": dict(zip(cfg.kinds, map(int, cal_ranges))),
                "mean_in_window_mse": dict(zip(cfg.kinds, map(float, cal_scores))),
                "wall_s": time.time() - t_cal,
            }
            log(f"calibrated ranges {calibration['ranges']} "
                f"(configured {dict(zip(cfg.kinds, cfg.ranges))})")

    peaks = None
    if not args.no_peaks:
        peaks = lib.measure_peaks(dev, stream)
        log("measured peaks: " + ", ".join(f"{k} {v:.0f}" for k, v in peaks.items()))

    # Per-type launch statistics over the timed trajectories' recomputes that
    # have a predecessor: the attention with the difference against that
    # predecessor folded into its output pass (where the kernel's LDS and the
    # workspace allow; else a separate pass inside the same bracket) and the
    # difference's final reduction.  Their algorithmic bytes add one read of
    # the previous output to the attention's own.
    kernels = {}
    for a, kind in enumerate(cfg.kinds):
        with_diff = [ev for ev, d in zip(brackets["attn"][a], brackets["diff"][a]) if d]
        st = stats_ms(with_diff or brackets["attn"][a])
        flops = harness.attn_flops(cfg, kind)
        by = harness.attn_bytes(cfg, kind) + (harness.mse_bytes(cfg) // 2 if with_diff else 0)
        st.update({
            "with_difference": bool(with_diff),
            "launches_per_trajectory": int(traj_on.counts[a]) * cfg.blocks,
            "flops_per_launch": flops,
            "bytes_per_launch": by,
            "tflops": flops / (st["mean_ms"] * 1e-3) / 1e12,
            "gbs": by / (st["mean_ms"] * 1e-3) / 1e9,
        })
        if kind == "spatial":
            st["frac_mfma"] = st["tflops"] / PEAK_BF16_TFLOPS
            if peaks:
                st["frac_mfma_measured_peak"] = st["tflops"] / peaks["mfma_bf16_tflops"]
        else:
            st["frac_hbm"] = st["gbs"] / PEAK_HBM_GBS
            if peaks:
                st["frac_hbm_measured_copy"] = st["gbs"] / peaks["hbm_copy_gbs"]
        st["traffic"] = read_traffic(cfg.name, kind)
        kernels[kind] = st
    # The standalone attention-difference MSE (pab_attn_diff_mse) on pairs of
    # cache slots, rotated so HBM serves them.  Inside the trajectory the
    # dispatcher folds the difference into the attention kernels' output
    # passes where its workspace holds their per-block partials.
    mse_ev = []
    pairs = [traj_on.slots[0][a] for a in range(len(cfg.kinds))]
    mse_out = torch.zeros(1, dtype=torch.float64, device=dev)
    for i in range(3 * len(pairs) + 1):
        x, y = pairs[i % len(pairs)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.pab_attn_diff_mse(x, y, mse_out, traj_on.ws, stream=stream.cuda_stream)
        e1.record(stream)
        if i > 0:  # the first launch loads the kernels
            mse_ev.append((e0, e1))
    torch.cuda.synchronize()
    st = stats_ms(mse_ev)
    if st:
        st.update({"bytes_per_launch": harness.mse_bytes(cfg),
                   "gbs": harness.mse_bytes(cfg) / (st["mean_ms"] * 1e-3) / 1e9})
        st["frac_hbm"] = st["gbs"] / PEAK_HBM_GBS
        if peaks:
            st["frac_hbm_measured_read"] = st["gbs"] / peaks["hbm_read_gbs"]
        st["traffic"] = read_traffic(cfg.name, "mse")
        kernels["mse"] = st

    flops_on = traj_on.flops()
    flops_off = traj_off.flops()
    value = flops_on / (on_ms * 1e-3) / 1e12

    # Roofline of the dominant kernel (spatial attention: bf16 MFMA).
    dom = "spatial"
    ach = kernels[dom]["tflops"]
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = read_traffic(cfg.name, dom)
    roofline = {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak, "traffic": traffic,
                "kernel": f"spatial_kernel<{cfg.D}>",
                "algorithmic_flops_per_launch": kernels[dom]["flops_per_launch"]}
    if peaks and cfg.dtype == "bf16":
        roofline["measured_peak"] = peaks["mfma_bf16_tflops"]
        roofline["frac_measured_peak"] = ach / peaks["mfma_bf16_tflops"]

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": on_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.desc + ", broadcast ranges "
                   + "/".join(f"{k} {r}" for k, r in zip(cfg.kinds, cfg.ranges))
                   + ", PAB on; one step = one whole trajectory: schedule, per-step "
                   "dispatch, and the attention-difference MSE after each recompute",
                   "name": cfg.name, "blocks": cfg.blocks, "denoise_steps": cfg.N,
                   "timing": ("sum of kernel brackets; inputs generated between dispatches"
                              if streamed else "trajectory wall time on the stream, inputs resident"),
                   "recomputes_per_type": dict(zip(cfg.kinds, map(int, traj_on.counts)))},
        "pab_on_ms_per_trajectory": on_ms,
        "pab_off_ms_per_trajectory": off_ms,
        "pab_on_without_mse_ms_per_trajectory": prod_ms,
        "range_calibration": calibration,
        "pab_speedup": (off_ms / on_ms) if off_ms else None,
        "effective_tflops_vs_off_work": flops_off / (on_ms * 1e-3) / 1e12,
        "pab_off_tflops": (flops_off / (off_ms * 1e-3) / 1e12) if off_ms else None,
        "kernels": kernels,
        "roofline": roofline,
        "measured_peaks": peaks,
    }
    if args.module_config:
        out["module"] = module_leg(args.module_config, args.module_steps, dev, stream)
        m = out["module"]
        log(f"modules {m['name']}: PAB on {m['pab_on_ms_per_trajectory']:.2f} ms, off "
            f"{m['pab_off_ms_per_trajectory']:.2f} ms; proj_in "
            f"{m['gemm']['proj_in']['tflops']:.0f} TFLOP/s, proj_out "
            f"{m['gemm']['proj_out']['tflops']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, traj_on, inputs, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
