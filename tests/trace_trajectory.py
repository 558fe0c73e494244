"""Runs small PAB trajectories on cuda:0 so that a kernel trace of this
process can be checked against the schedule; started by
``test_gpu_zz_launch_trace.py`` under ``rocprofv3 --kernel-trace``.

It prints one JSON line, ``expected``: how many launches of each kernel the
trajectories must make, derived from the oracle's schedule (recomputes per
type, PAB article, Implementation and Figure 2 caption) and the launch
rules of the dispatcher:
- a recompute of a bf16 attention launches its kernel once (a padded-prompt
  cross attention once per batch entry); with the attention difference on,
  every recompute that has a predecessor adds one final reduction, and the
  partial sums come from the attention launch itself;
- an fp32 recompute launches the fp32 attention kernel once, and the
  difference is a separate pass (partial and final reduction);
- an attention module launches the input projection (a cross module a
  second one for the text), the attention and the output projection, and
  the difference of the module output is a separate pass;
- a broadcast step launches nothing.
The last line printed is ``trace-run done``.
"""

import dataclasses
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch  # noqa: E402

import oracle  # noqa: E402
from reuse_pab_plan_amd import harness, lib  # noqa: E402

KINDS = ("spatial", "temporal", "cross")


def workloads():
    base = harness.Config("trace_bf16", "bf16", 1, 2, 8, 300, 72, 16, 12, KINDS, (2, 3, 5), 3, 41,
                          "launch-count trace: 3 blocks, 8 frames x 300 tokens")
    return [
        (base, True),
        (dataclasses.replace(base, name="trace_bf16_off", blocks=1, seed=42), False),
        (dataclasses.replace(base, name="trace_cfg", B=2, blocks=1, seed=43, text_len=(7, 1),
                             const_text=True), True),
        (harness.CONFIGS["tiny"], True),
        (harness.CONFIGS["mod_small"], True),
    ]


def expected_launches(cfg, pab):
    ranges = list(cfg.ranges) if pab else [0] * len(cfg.kinds)
    _, _, counts = oracle.schedule(cfg.N, ranges)
    e = {}

    def add(name, n):
        e[name] = e.get(name, 0) + int(n)

    for a, kind in enumerate(cfg.kinds):
        rec = int(counts[a]) * cfg.blocks
        diffs = max(int(counts[a]) - 1, 0) * cfg.blocks  # recomputes with a predecessor
        if cfg.module:
            add("proj_in", rec * (2 if kind == "cross" else 1))
            add("proj_out", rec)
            add(kind, rec)
            add("mse_partial", diffs)
        elif cfg.dtype == "f32":
            add("attn_f32", rec)
            add("mse_partial", diffs)
        else:
            parts = cfg.B if (kind == "cross" and cfg.text_len
                              and any(t != cfg.L for t in cfg.text_len)) else 1
            add(kind, rec * parts)
        add("mse_final", diffs)
    return e


def main():
    lib.load()
    dev = torch.device("cuda:0")
    total = {}
    for cfg, pab in workloads():
        print(f"[trace] {cfg.name} pab={pab}", flush=True)
        traj = harness.Trajectory(cfg, pab=pab, device=dev)
        traj.inputs = harness.Inputs(cfg, traj.steps_needed(), device=dev, resident=True)
        torch.cuda.synchronize()
        traj.run()
        torch.cuda.synchronize()
        for k, v in expected_launches(cfg, pab).items():
            total[k] = total.get(k, 0) + v
    print("expected " + json.dumps(total, sort_keys=True), flush=True)
    print("trace-run done", flush=True)


if __name__ == "__main__":
    main()
