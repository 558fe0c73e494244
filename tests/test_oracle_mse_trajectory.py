"""Pins for oracle.mse and oracle.trajectory.

MSE: a hand-computed example, identities and exact dyadic shifts.
Trajectory: PAB off reproduces per-step attention; reuse hands back the
source step's output unchanged; the evaluation count equals the closed-form
recompute count; the synthetic workload shows the U shape qualitatively.
"""

import numpy as np
import pytest

from oracle import attn_fp64, closed_form_counts, cross, mse, spatial, temporal, trajectory
from reuse_pab_plan_amd import synth


def test_mse_hand_example():
    assert mse([1.0, 2.0, 3.0], [1.0, 0.0, 0.0]) == pytest.approx(13.0 / 3.0, rel=0, abs=1e-15)


def test_mse_identities():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(1001).astype(np.float32)
    y = rng.standard_normal(1001).astype(np.float32)
    assert mse(x, x) == 0.0
    assert mse(x, y) == mse(y, x)
    assert mse(x, y) > 0.0
    ints = rng.integers(-1000, 1000, 4097).astype(np.float32)
    assert mse(ints, ints + np.float32(0.5)) == 0.25       # exact
    assert mse(ints, ints - np.float32(3.0)) == 9.0         # exact
    assert mse([2.5], [0.5]) == 4.0


def test_mse_rejects_bad_sizes():
    with pytest.raises(ValueError):
        mse([1.0], [1.0, 2.0])
    with pytest.raises(ValueError):
        mse([], [])


SHAPE = (1, 2, 3, 8, 8)   # B H F S D
TEXT = (1, 2, 5, 8)
KINDS = ["spatial", "temporal", "cross"]


def make_inputs(n_steps, seed=11):
    cache = {}

    def fn(step, a):
        key = (step, a)
        if key not in cache:
            qshape = SHAPE
            kshape = TEXT if KINDS[a] == "cross" else SHAPE
            cache[key] = {
                "q": synth.cpu_tensor(qshape, seed, 0, a, 0, step, n_steps).numpy(),
                "k": synth.cpu_tensor(kshape, seed, 0, a, 1, step, n_steps).numpy(),
                "v": synth.cpu_tensor(kshape, seed, 0, a, 2, step, n_steps).numpy(),
            }
        return cache[key]

    return fn


def direct(kind, x):
    return {"spatial": spatial, "temporal": temporal, "cross": cross}[kind](x["q"], x["k"], x["v"])


def test_pab_off_is_per_step_attention():
    n = 10
    fn = make_inputs(n)
    res = trajectory(n, KINDS, [0, 0, 0], fn)
    assert res["calls"] == 3 * n
    for i in range(n):
        for a, kind in enumerate(KINDS):
            assert np.array_equal(res["outputs"][i][a], direct(kind, fn(i, a)))


def test_pab_on_reuses_source_outputs():
    n = 10
    ranges = [2, 3, 5]
    fn = make_inputs(n)
    res = trajectory(n, KINDS, ranges, fn)
    assert res["calls"] == int(closed_form_counts(n, ranges).sum()) == 16
    for i in range(n):
        for a, kind in enumerate(KINDS):
            j = res["source"][i][a]
            assert res["outputs"][i][a] is res["outputs"][j][a]
            assert np.array_equal(res["outputs"][i][a], direct(kind, fn(j, a)))


def test_drift_is_mse_between_successive_computations():
    n = 10
    fn = make_inputs(n)
    res = trajectory(n, KINDS, [2, 3, 5], fn)
    for a in range(3):
        computed = [i for i in range(n) if res["recompute"][i][a]]
        assert res["drift"][computed[0]][a] is None
        for prev, cur in zip(computed, computed[1:]):
            expect = mse(res["outputs"][cur][a], res["outputs"][prev][a])
            assert res["drift"][cur][a] == expect


def test_u_shape_on_synthetic_workload():
    # Qualitative harness check: consecutive-step differences (PAB off) are
    # larger on the outer steps than in the middle, as the PAB article's
    # first observation describes for real models.
    n = 20
    fn = make_inputs(n, seed=3)
    res = trajectory(n, KINDS, [0, 0, 0], fn)
    for a in range(3):
        d = [res["drift"][i][a] for i in range(1, n)]
        inner = [d[i - 1] for i in range(5, 17)]      # both ends inside
        outer = [d[0], d[1], d[2], d[-1], d[-2]]
        assert min(outer) > 10 * max(inner)


def test_synth_streams_distinct_and_deterministic():
    a = synth.cpu_tensor((4, 4), 1, 0, 0, 0, 3, 10).numpy()
    b = synth.cpu_tensor((4, 4), 1, 0, 0, 0, 3, 10).numpy()
    c = synth.cpu_tensor((4, 4), 1, 0, 0, 1, 3, 10).numpy()
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert synth.step_sigma(0, 30) == 0.5 and synth.step_sigma(5, 30) == 0.02
    assert synth.step_sigma(25, 30) == 0.02 and synth.step_sigma(26, 30) == 0.5


def test_attn_used_by_trajectory_is_the_definition():
    x = make_inputs(3)(0, 0)
    assert np.array_equal(direct("spatial", x), attn_fp64(x["q"], x["k"], x["v"]))


def test_trajectory_custom_compute_is_called_at_recomputes_only():
    # A compute function replaces the attention (an attention module, say):
    # it runs exactly at recompute steps, and every output is the one of the
    # step's source.
    seen = []

    def compute(kind, x):
        seen.append((x["step"], kind))
        return np.array([x["step"]])

    res = trajectory(12, ["spatial", "cross"], [2, 4],
                            lambda i, a: {"step": i}, compute=compute)
    rec, src = res["recompute"], res["source"]
    assert sorted(seen) == sorted((i, k) for i in range(12) for a, k in enumerate(["spatial", "cross"])
                                  if rec[i, a])
    for i in range(12):
        for a in range(2):
            assert int(res["outputs"][i][a][0]) == int(src[i, a])
