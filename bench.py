#!/usr/bin/env python3
"""Benchmark of the PAB attention hot path on one MI355X.

One benchmark step is one whole denoising trajectory of the headline
workload, by default the 28-block stack at the 480p-latent shape (per block:
48 frames x 1590 tokens, 16 heads x 72, 120 text tokens; 30 steps; broadcast
ranges spatial 2 / temporal 4 / cross 6; bf16): the schedule from
pab_plan_schedule, then per step and block pab_step_dispatch for each
attention type (spatial, temporal and cross kernels on recompute steps,
nothing on broadcast steps; the 28 x 3 x 2 cache slots stay in HBM), each
recompute also taking the attention-difference MSE against the previous
computation of its type (the quantity the pages plot to motivate the
broadcast ranges, used to calibrate them; the dispatcher folds it into the
attention kernels' output pass).

Inputs: a workload whose inputs fit in HBM has every step's inputs generated
before timing, and a step is timed as the trajectory's wall time on the
stream.  The stack's inputs (about 0.5 TB over a trajectory) do not fit: they
are drawn by the library's device generator one recompute ahead, between the
dispatches, and a step is timed as the sum of HIP-event brackets around the
dispatches (the generator runs outside them); the wall time including
generation is reported beside it.

Prints one JSON line: metric, value (attention TFLOP/s executed per second
of PAB-on trajectory), ms_per_step (ms per PAB-on trajectory), the PAB-off
trajectory beside it, per-kernel timings, the roofline of the dominant
kernel (spatial attention, bf16 MFMA) measured live with HIP events on the
launch stream, the extra workloads (b480, b720, full3d) as keys of their
own, and the CPU oracle timed on the host.

    python bench.py [--steps K] [--warmup W] [--config stack28|b480|b720|full3d|cfg480|tiny]
                    [--extra-configs b480,b720,full3d] [--module-config b480m|""]
                    [--stream-inputs] [--no-peaks] [--no-cpu-baseline] [--calib-copy]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

# The oracle's BLAS uses the cores this process may run on (unless the
# environment already says otherwise); set before numpy is first imported.
_AFFINITY = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
    os.environ.setdefault(_var, str(_AFFINITY))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and ms per denoise trajectory (PAB on/off), % of roofline"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_b480.md")
# Workloads whose kernels run at another workload's per-launch shape.
SAME_SHAPE = {"stack28": "b480"}
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
    the summary is missing, is for another launch shape, or was taken on a
    different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    tr = json.loads(text[start + 7:end])
    k = tr.get("kernels", {}).get(kernel)
    shape = SAME_SHAPE.get(config, config)
    if tr.get("config") != shape or not k or k.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return k.get("hbm_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed PAB-on trajectories")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--off-steps", type=int, default=3, help="timed PAB-off trajectories")
    ap.add_argument("--config", default="stack28")
    ap.add_argument("--extra-configs", default="b480,b720,full3d",
                    help="workloads timed after the headline, each under its own key ('' to skip)")
    ap.add_argument("--extra-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--module-config", default="b480m",
                    help="attention-module workload timed after the main line ('' to skip)")
    ap.add_argument("--module-steps", type=int, default=3)
    ap.add_argument("--stream-inputs", action="store_true",
                    help="draw each recompute's inputs between the dispatches even when the "
                         "workload's inputs would fit in HBM")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the sustained-peak microbenchmarks (measured roofline denominators)")
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="seconds of oracle work at most (the headline step is sampled past it)")
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


def inputs_fit(cfg, free_bytes):
    """Whether every input of a PAB-off trajectory fits in HBM beside the cache."""
    from reuse_pab_plan_amd import harness

    per = {"spatial": 3, "temporal": 3, "cross": 1}
    n = cfg.B * cfg.H * cfg.F * cfg.S * cfg.D * cfg.elem_bytes
    need = cfg.blocks * cfg.N * sum(per[k] for k in cfg.kinds) * n + harness.cache_bytes(cfg)
    return need < 0.6 * free_bytes


# ------------------------------------------------------------------ CPU oracle

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, traj_on, inputs, budget_s):
    """Time the oracle (as it stands) on the host cores.

    * tiny: the whole fp32 trajectory through ``oracle.trajectory`` with
      ``attn_fp64``, PAB on and off; one step of every type with the literal
      loops of ``attn_loop`` (pure Python: one core);
    * the headline workload: one full step of each attention type at its
      per-block shape (spatial sampled by whole heads only if the budget
      runs out), and one oracle MSE on two output-sized tensors.  Every call
      of a type has the same shape and cost, so the trajectory time is
      derived as blocks x sum_a count_a x t_a + (MSE calls) x t_mse;
    * b720 and full3d: each type's call time from a sample (a quarter of the
      query rows of one sequence for spatial, one (b, h) for temporal and
      cross), and their trajectory times derived the same way.
    """
    import numpy as np
    import threadpoolctl

    import oracle
    from reuse_pab_plan_amd import harness, synth

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] + [1])
    t_start = time.perf_counter()
    legs = {}

    # tiny, PAB on and off (fp32 inputs drawn on the host, same shapes)
    tiny = harness.CONFIGS["tiny"]
    t_in = {}

    def tiny_inputs(i, a):
        if (i, a) not in t_in:
            kind = tiny.kinds[a]
            kv = tiny.text_shape if kind == "cross" else tiny.video_shape
            t = harness.TYPE_INDEX[kind]
            t_in[(i, a)] = {"q": synth.cpu_tensor(tiny.video_shape, tiny.seed, 0, t, 0, i, tiny.N).numpy(),
                            "k": synth.cpu_tensor(kv, tiny.seed, 0, t, 1, i, tiny.N).numpy(),
                            "v": synth.cpu_tensor(kv, tiny.seed, 0, t, 2, i, tiny.N).numpy()}
        return t_in[(i, a)]

    for i in range(tiny.N):
        for a in range(len(tiny.kinds)):
            tiny_inputs(i, a)
    for label, ranges in (("pab_on", list(tiny.ranges)), ("pab_off", [0] * len(tiny.kinds))):
        t0 = time.perf_counter()
        oracle.trajectory(tiny.N, list(tiny.kinds), ranges, tiny_inputs)
        legs[f"tiny_trajectory_{label}_ms"] = (time.perf_counter() - t0) * 1e3
    # literal loops, one step of every type (one core: pure Python)
    x = tiny_inputs(0, 0)
    t0 = time.perf_counter()
    q, k, v = x["q"], x["k"], x["v"]
    for b in range(tiny.B):
        for h in range(tiny.H):
            for f in range(tiny.F):
                oracle.attn_loop(q[b, h, f], k[b, h, f], v[b, h, f])
    legs["tiny_spatial_step_attn_loop_ms"] = (time.perf_counter() - t0) * 1e3
    x = tiny_inputs(0, 1)
    q, k, v = x["q"], x["k"], x["v"]
    t0 = time.perf_counter()
    for b in range(tiny.B):
        for h in range(tiny.H):
            for s in range(tiny.S):
                oracle.attn_loop(q[b, h, :, s], k[b, h, :, s], v[b, h, :, s])
    legs["tiny_temporal_step_attn_loop_ms"] = (time.perf_counter() - t0) * 1e3
    x = tiny_inputs(0, 2)
    q, k, v = x["q"], x["k"], x["v"]
    t0 = time.perf_counter()
    for b in range(tiny.B):
        for h in range(tiny.H):
            oracle.attn_loop(q[b, h].reshape(-1, tiny.D), k[b, h], v[b, h])
    legs["tiny_cross_step_attn_loop_ms"] = (time.perf_counter() - t0) * 1e3

    # b720 and full3d: the oracle's time per call of each type from a sample
    # (a quarter of the query rows of one frame-sequence for spatial, one
    # (b, h) for temporal and cross),
    # scaled to a whole call (every sequence of a call has the same shape and
    # cost); their trajectory times are derived as for the headline, the
    # MSE scaled by its element count from the headline's.
    derived = {}
    for name in ("b720", "full3d"):
        c2 = harness.CONFIGS[name]
        per = {}
        for a, kind in enumerate(c2.kinds):
            t = harness.TYPE_INDEX[kind]
            if kind == "spatial":
                shp, kv, share = (1, 1, 1, c2.S, c2.D), (1, 1, 1, c2.S, c2.D), c2.B * c2.H * c2.F
            elif kind == "temporal":
                shp, kv, share = (1, 1, c2.F, c2.S, c2.D), (1, 1, c2.F, c2.S, c2.D), c2.B * c2.H
            else:
                shp, kv, share = (1, 1, c2.F, c2.S, c2.D), (1, 1, c2.L, c2.D), c2.B * c2.H
            q = synth.cpu_tensor(shp, c2.seed, 0, t, 0, 0, c2.N).numpy()
            k = synth.cpu_tensor(kv, c2.seed, 0, t, 1, 0, c2.N).numpy()
            v = synth.cpu_tensor(kv, c2.seed, 0, t, 2, 0, c2.N).numpy()
            t0 = time.perf_counter()
            if kind == "spatial":  # a quarter of the query rows of the sequence
                rows = np.arange(0, c2.S, 4)
                oracle.spatial_rows(q, k, v, 0, 0, 0, rows)
                share *= c2.S / len(rows)
            else:
                getattr(oracle, kind)(q, k, v)
            per[kind] = (time.perf_counter() - t0) * share * 1e3
        derived[name] = {"per_call_ms": per, "counts": dict(zip(c2.kinds, map(
            int, oracle.schedule(c2.N, list(c2.ranges))[2])))}

    # The headline workload, per block: one full step of each type.
    rates, per_call, sample = [], {}, []
    per_type = max(budget_s - (time.perf_counter() - t_start), 5.0) / len(cfg.kinds)
    for a, kind in enumerate(cfg.kinds):
        q, k, v = inputs.get(0, a, 0)
        done_flops, t_used, heads = 0, 0.0, 0
        for b in range(cfg.B):
            for h in range(cfg.H):
                qh = q[b:b + 1, h:h + 1].float().cpu().numpy()
                kh = k[b:b + 1, h:h + 1].float().cpu().numpy()
                vh = v[b:b + 1, h:h + 1].float().cpu().numpy()
                t0 = time.perf_counter()
                getattr(oracle, kind)(qh, kh, vh)
                t_used += time.perf_counter() - t0
                heads += 1
                done_flops += harness.attn_flops(cfg, kind) // (cfg.B * cfg.H)
                if t_used >= per_type and heads < cfg.B * cfg.H:
                    break
            else:
                continue
            break
        rates.append(done_flops / t_used)
        per_call[kind] = harness.attn_flops(cfg, kind) / rates[-1] * 1e3
        whole = heads == cfg.B * cfg.H
        sample.append(f"{kind}: {'the whole step' if whole else f'{heads} of {cfg.B * cfg.H} heads'}"
                      f" ({t_used:.1f} s)")
    q0, k0, _ = inputs.get(0, 0, 0)  # two tensors of the output's size
    o1, o2 = q0.float().cpu().numpy(), k0.float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.mse(o1, o2)
    mse_s = time.perf_counter() - t0
    n_mse = sum(max(int(traj_on.counts[a]) - 1, 0) for a in range(len(cfg.kinds))) * cfg.blocks
    sample.append(f"mse: one call on two output-sized tensors ({mse_s * 1e3:.0f} ms)")
    traj_s = sum(int(traj_on.counts[a]) * harness.attn_flops(cfg, kind) * cfg.blocks / rates[a]
                 for a, kind in enumerate(cfg.kinds)) + n_mse * mse_s
    n_head = cfg.B * cfg.H * cfg.F * cfg.S * cfg.D
    for name, dv in derived.items():
        c2 = harness.CONFIGS[name]
        mse_ms = mse_s * 1e3 * (c2.B * c2.H * c2.F * c2.S * c2.D) / n_head
        n2 = sum(max(c - 1, 0) for c in dv["counts"].values())
        legs[f"{name}_per_call_ms_derived"] = dv["per_call_ms"]
        legs[f"{name}_trajectory_pab_on_ms_derived"] = (
            sum(dv["counts"][k] * dv["per_call_ms"][k] for k in dv["counts"]) + n2 * mse_ms)
    value = traj_on.flops() / traj_s / 1e12
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"per-block step of each type at the {cfg.name} shape: " + "; ".join(sample)
                  + f"; fp64 numpy oracle; trajectory time derived as blocks x sum of count x "
                  f"per-call time = {traj_s:.1f} s per PAB-on trajectory; attn_loop legs are "
                  f"pure Python on one core",
        "ms_per_trajectory": traj_s * 1e3,
        "per_call_ms": per_call,
        "legs": legs,
        "cpu_model": cpu_model(),
        "blas_threads": int(threads),
        "env_threads": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")},
        "host_cpus": os.cpu_count(),
        "affinity_cpus": _AFFINITY,
        "wall_s": time.perf_counter() - t_start,
    }


# ---------------------------------------------------------- trajectory legs

def trajectory_leg(cfg, steps, warmup, off_steps, streamed, dev, stream, peaks=None,
                   calibrate=True):
    """PAB on (with and without the attention difference) and PAB off over
    one workload.  Returns (result dict, PAB-on trajectory, inputs)."""
    import numpy as np
    import torch

    from reuse_pab_plan_amd import harness, lib

    traj_on = harness.Trajectory(cfg, pab=True, device=dev, stream=stream, drift=False)
    traj_off = harness.Trajectory(cfg, pab=False, device=dev, stream=stream, drift=False)
    t0 = time.time()
    needed = traj_off.steps_needed() if off_steps > 0 else traj_on.steps_needed()
    inputs = harness.Inputs(cfg, [] if streamed else needed, device=dev, resident=not streamed)
    traj_on.inputs = inputs
    traj_off.inputs = inputs
    torch.cuda.synchronize()
    log(f"{cfg.name}: inputs {'drawn per recompute' if streamed else 'resident'} "
        f"({time.time() - t0:.1f}s, {torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")

    def timed(traj, n):
        """n trajectories: (wall ms, kernel-bracket ms, brackets) per trajectory."""
        br = {"attn": [[] for _ in cfg.kinds], "diff": [[] for _ in cfg.kinds]}
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        last = None
        for _ in range(n):
            traj.replan()
            last = traj.run(events=True)
            for a in range(len(cfg.kinds)):
                br["attn"][a] += last["brackets"]["attn"][a]
                br["diff"][a] += last["brackets"]["diff"][a]
        stop.record(stream)
        torch.cuda.synchronize()
        wall = start.elapsed_time(stop) / n
        kern = sum(a.elapsed_time(b) for v in br["attn"] for a, b in v) / n
        return wall, kern, br, last

    # One bench step is one pass of the whole path: plan the schedule, then
    # the PAB-on trajectory -- each step's dispatch (attention kernels on
    # recompute steps, the cache slot in place on broadcast steps) and, after
    # each recompute, the attention-difference MSE against the previous
    # computation of its type (Figure 1's quantity).
    traj_on.drift = True
    for _ in range(warmup):
        traj_on.replan()
        traj_on.run(events=False)
    torch.cuda.synchronize()
    wall, kern, brackets, r = timed(traj_on, steps)
    on_ms = kern if streamed else wall
    log(f"{cfg.name} PAB on (schedule, dispatch, attention-difference MSE): {on_ms:.3f} ms per "
        f"trajectory ({'kernel brackets' if streamed else 'wall'}; wall {wall:.1f} ms)")
    for a in range(len(cfg.kinds)):
        for b in range(cfg.blocks):
            got = (r["masks"][b] >> a) & 1
            if not (got == traj_on.recompute[:, a]).all():
                raise RuntimeError(f"dispatch mask of block {b}, type {a} differs from the schedule")

    # The same trajectory as a production run would take it: no MSE.
    traj_on.drift = False
    n_prod = max(1, min(steps, 5))
    p_wall, p_kern, _, _ = timed(traj_on, n_prod)
    prod_ms = p_kern if streamed else p_wall
    log(f"{cfg.name} PAB on without the MSE: {prod_ms:.3f} ms per trajectory")

    # The PAB-on trajectory (with the MSE) recorded once as a HIP graph and
    # replayed: the same device work with one host call per trajectory
    # (resident inputs only; the schedule is the one planned at capture).
    graph_ms = None
    if not streamed:
        traj_on.drift = True
        traj_on.replan()
        graph, _ = traj_on.capture()
        with torch.cuda.stream(stream):
            graph.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        n_g = max(1, min(steps, 10))
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(n_g):
                graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / n_g
        del graph
        log(f"{cfg.name} PAB on replayed from a HIP graph: {graph_ms:.3f} ms per trajectory")

    off_ms, off_wall, calibration = None, None, None
    if off_steps > 0:
        # PAB off, the same pass (schedule, every step computed, MSE).
        traj_off.drift = True
        traj_off.run(events=False)
        o_wall, o_kern, _, _ = timed(traj_off, off_steps)
        traj_off.drift = False
        off_ms, off_wall = (o_kern if streamed else o_wall), o_wall
        log(f"{cfg.name} PAB off (schedule, dispatch, MSE): {off_ms:.3f} ms per trajectory")
        if calibrate:
            # Range calibration from the PAB-off trajectories' attention
            # difference (every block; the planner averages them).
            t_cal = time.time()
            cal_ranges, cal_scores, _ = harness.calibrate(traj_off, rerun=False)
            calibration = {
                "candidates": list(cfg.ranges),
                "ranges": dict(zip(cfg.kinds, map(int, cal_ranges))),
                "mean_in_window_mse": dict(zip(cfg.kinds, map(float, cal_scores))),
                "blocks": cfg.blocks,
                "wall_s": time.time() - t_cal,
            }
            log(f"{cfg.name} calibrated ranges {calibration['ranges']} "
                f"(configured {dict(zip(cfg.kinds, cfg.ranges))})")

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
            peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
            st["frac_mfma" if cfg.dtype == "bf16" else "frac_f32"] = st["tflops"] / peak
            if peaks and cfg.dtype == "bf16":
                st["frac_mfma_measured_peak"] = st["tflops"] / peaks["mfma_bf16_tflops"]
        else:
            st["frac_hbm"] = st["gbs"] / PEAK_HBM_GBS
            if peaks:
                # against the measured stream rate of the kernel's own
                # read:write mix (previous output read when fused)
                mix = {"temporal": "4:1" if with_diff else "3:1",
                       "cross": "2:1" if with_diff else "1:1"}[kind]
                st["hbm_mix"] = mix
                st["frac_hbm_measured"] = st["gbs"] / peaks["hbm_stream_gbs"][mix]
        st["traffic"] = read_traffic(cfg.name, kind)
        kernels[kind] = st
    # The standalone attention-difference MSE (pab_attn_diff_mse) on pairs of
    # cache slots of different blocks, rotated so HBM serves them.
    mse_ev = []
    pairs = [traj_on.slots[b][a] for b in range(min(cfg.blocks, 4)) for a in range(len(cfg.kinds))]
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
            st["hbm_mix"] = "2:0"
            st["frac_hbm_measured"] = st["gbs"] / peaks["hbm_stream_gbs"]["2:0"]
        st["traffic"] = read_traffic(cfg.name, "mse")
        kernels["mse"] = st

    flops_on = traj_on.flops()
    flops_off = traj_off.flops()
    res = {
        "workload": cfg.desc,
        "name": cfg.name,
        "blocks": cfg.blocks,
        "timing": ("sum of HIP-event brackets around the dispatches; inputs drawn by the device "
                   "generator between them" if streamed
                   else "trajectory wall time on the stream, inputs resident in HBM"),
        "recomputes_per_type": dict(zip(cfg.kinds, map(int, traj_on.counts))),
        "pab_on_ms_per_trajectory": on_ms,
        "pab_on_wall_ms_per_trajectory": wall,
        "pab_on_without_mse_ms_per_trajectory": prod_ms,
        "pab_on_graph_replay_ms_per_trajectory": graph_ms,
        "pab_off_ms_per_trajectory": off_ms,
        "pab_off_wall_ms_per_trajectory": off_wall,
        "pab_speedup": (off_ms / on_ms) if off_ms else None,
        "tflops_pab_on": flops_on / (on_ms * 1e-3) / 1e12,
        "effective_tflops_vs_off_work": flops_off / (on_ms * 1e-3) / 1e12,
        "pab_off_tflops": (flops_off / (off_ms * 1e-3) / 1e12) if off_ms else None,
        "range_calibration": calibration,
        "kernels": kernels,
    }
    del traj_off
    return res, traj_on, inputs


def module_leg(name, steps, dev, stream):
    """Attention modules (input projection, attention, output projection
    around each attention type) over a PAB-on and a PAB-off trajectory, and
    the two projection GEMMs timed alone at the workload's shapes."""
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

    import torch

    from reuse_pab_plan_amd import harness, lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib.load()
    cfg = harness.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)

    if args.calib_copy:
        # Plain copy of exactly 2 GiB read + 2 GiB written, for scaling the
        # FETCH_SIZE / WRITE_SIZE counters of the attention kernels.
        src = torch.empty(2**30, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    peaks = None
    if not args.no_peaks:
        peaks = lib.measure_peaks(dev, stream)
        log("measured peaks: " + ", ".join(f"{k} {v:.0f}" for k, v in peaks.items()
                                           if isinstance(v, float))
            + "; streams GB/s " + ", ".join(f"{k} {v:.0f}" for k, v in peaks["hbm_stream_gbs"].items()))

    streamed = args.stream_inputs or not inputs_fit(cfg, torch.cuda.mem_get_info(dev)[0])
    head, traj_on, inputs = trajectory_leg(cfg, args.steps, args.warmup, args.off_steps, streamed,
                                           dev, stream, peaks)
    on_ms = head["pab_on_ms_per_trajectory"]
    value = traj_on.flops() / (on_ms * 1e-3) / 1e12
    kernels = head["kernels"]

    # Roofline of the dominant kernel (spatial attention: bf16 MFMA).
    dom = "spatial"
    ach = kernels[dom]["tflops"]
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    roofline = {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak, "traffic": read_traffic(cfg.name, dom),
                "kernel": f"spatial_kernel<{cfg.D}>",
                "algorithmic_flops_per_launch": kernels[dom]["flops_per_launch"],
                "launches_timed": kernels[dom]["n"]}
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
                   "timing": head["timing"],
                   "recomputes_per_type": head["recomputes_per_type"]},
        "roofline": roofline,
    }
    for key in ("pab_on_ms_per_trajectory", "pab_on_wall_ms_per_trajectory",
                "pab_on_without_mse_ms_per_trajectory", "pab_on_graph_replay_ms_per_trajectory",
                "pab_off_ms_per_trajectory",
                "pab_off_wall_ms_per_trajectory", "pab_speedup", "effective_tflops_vs_off_work",
                "pab_off_tflops", "range_calibration", "kernels"):
        out[key] = head[key]
    out["measured_peaks"] = peaks

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, traj_on, inputs, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    del traj_on, inputs
    torch.cuda.empty_cache()

    # The other single-block workloads, each under its own key.
    extra = {}
    for name in [n for n in args.extra_configs.split(",") if n and n != cfg.name]:
        ecfg = harness.CONFIGS[name]
        ex_stream = args.stream_inputs or not inputs_fit(ecfg, torch.cuda.mem_get_info(dev)[0])
        res, t_on, t_in = trajectory_leg(ecfg, args.extra_steps, 2, 2, ex_stream, dev, stream,
                                         peaks, calibrate=False)
        extra[name] = res
        del t_on, t_in
        torch.cuda.empty_cache()
    out["workloads"] = extra

    if args.module_config:
        out["module"] = module_leg(args.module_config, args.module_steps, dev, stream)
        m = out["module"]
        log(f"modules {m['name']}: PAB on {m['pab_on_ms_per_trajectory']:.2f} ms, off "
            f"{m['pab_off_ms_per_trajectory']:.2f} ms; proj_in "
            f"{m['gemm']['proj_in']['tflops']:.0f} TFLOP/s, proj_out "
            f"{m['gemm']['proj_out']['tflops']:.0f} TFLOP/s")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
