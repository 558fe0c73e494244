"""GPU tests of a whole PAB trajectory recorded as one HIP graph and replayed.

The schedule fixes every launch of a trajectory (PAB article, Figure 2
caption: an attention is recomputed on schedule steps and broadcast to the
following ones), so the trajectory can be captured once and replayed.  Each
replay must leave every cache slot and the drift record bit-identical to the
eager run of the same trajectory -- the kernels are deterministic -- replay
after replay, with other device work and host synchronizations between the
replays, and with the outputs overwritten before each replay so that a
replay that skipped a launch would show.
"""

import dataclasses

import pytest
import torch

from reuse_pab_plan_amd import harness, lib

pytestmark = pytest.mark.gpu

KINDS = ("spatial", "temporal", "cross")
BF16 = harness.Config("graph_bf16", "bf16", 1, 2, 8, 300, 72, 16, 12, KINDS, (2, 3, 5), 3, 51,
                      "graph replay: 3 blocks, 8 frames x 300 tokens")
CASES = {
    "tiny": harness.CONFIGS["tiny"],
    "bf16_3blocks": BF16,
    "bf16_padded_prompt": dataclasses.replace(BF16, name="graph_cfg", B=2, blocks=1, seed=52,
                                              text_len=(7, 1), const_text=True),
    "mod_small": harness.CONFIGS["mod_small"],
}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()


def _fingerprint(t):
    """Exact content fingerprint of a device tensor (int64 sums of the bits)."""
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16)
    elif t.dtype == torch.float64:
        bits = t.view(torch.int64)
    else:
        bits = t.view(torch.int32)
    x = bits.to(torch.int64).flatten()
    idx = torch.arange(x.numel(), device=x.device, dtype=torch.int64)
    return (int(x.sum()), int((x * (idx % 65521 + 1)).sum()))


def _clobber(traj):
    """Overwrite every cache slot (NaN) and the drift record (-1)."""
    for row in traj.slots:
        for s0, s1 in row:
            s0.fill_(float("nan"))
            s1.fill_(float("nan"))
    traj.drift_out.fill_(-1.0)


def _state(traj):
    torch.cuda.synchronize()
    return ([[(_fingerprint(s0), _fingerprint(s1)) for s0, s1 in row] for row in traj.slots],
            _fingerprint(traj.drift_out))


RUNS = [(name, True, True) for name in CASES] + [("tiny", False, True), ("bf16_3blocks", True, False)]


@pytest.mark.parametrize("name,pab,drift", RUNS,
                         ids=[f"{n}-{'pab' if p else 'off'}-{'drift' if d else 'nodrift'}"
                              for n, p, d in RUNS])
def test_graph_replay_matches_eager(name, pab, drift):
    _need_gpu()
    cfg = CASES[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    print(f"[graph] {name} pab={pab} drift={drift}", flush=True)
    traj = harness.Trajectory(cfg, pab=pab, device=dev, stream=stream, drift=drift)
    traj.inputs = harness.Inputs(cfg, traj.steps_needed(), device=dev, resident=True)
    _clobber(traj)
    rec_eager = traj.run()
    ref = _state(traj)
    untouched = _fingerprint(torch.full_like(traj.drift_out, -1.0))
    if drift:
        assert ref[1] != untouched, "no drift was taken"
    else:
        assert ref[1] == untouched, "drift written with the difference off"

    graph, rec_cap = traj.capture()
    # The captured pass made the same host-side decisions as the eager one.
    assert (rec_cap["masks"] == rec_eager["masks"]).all()
    assert rec_cap["outs"] == rec_eager["outs"]

    other = torch.empty(1 << 20, device=dev)
    for rep in range(3):
        _clobber(traj)
        other.normal_()  # unrelated eager work between the replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        got = _state(traj)
        print(f"[graph] {name} replay {rep}: identical={got == ref}", flush=True)
        assert got == ref, (name, rep)


def test_capture_needs_resident_inputs_and_a_side_stream():
    _need_gpu()
    cfg = harness.CONFIGS["tiny"]
    dev = torch.device("cuda:0")
    traj = harness.Trajectory(cfg, pab=True, device=dev, stream=torch.cuda.Stream(dev))
    traj.inputs = harness.Inputs(cfg, traj.steps_needed(), device=dev, resident=False)
    with pytest.raises(ValueError, match="resident"):
        traj.capture()
    traj2 = harness.Trajectory(cfg, pab=True, device=dev,
                               stream=torch.cuda.default_stream(dev))
    traj2.inputs = harness.Inputs(cfg, traj2.steps_needed(), device=dev, resident=True)
    with pytest.raises(ValueError, match="default stream"):
        traj2.capture()
