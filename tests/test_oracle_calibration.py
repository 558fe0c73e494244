"""Range calibration (oracle and the C planner) pinned to hand-worked cases.

The oracle's ``calibrate_ranges`` is checked against cases worked by hand
from the pages (tests/golden/calibration_cases.txt), and against properties
the rule must have whatever its implementation: ranges only depend on the
order of the scores (scaling every difference by a power of two changes
nothing), relabelling the types relabels the ranges, and steps outside the
stable window never matter.  The C entry point ``pab_plan_calibrate`` must
then agree with the oracle bit for bit (ranges) and exactly (scores: the
same fp64 sums in the same order).
"""

import ctypes as C
import math
import os

import numpy as np
import pytest

import oracle
from reuse_pab_plan_amd import lib

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "calibration_cases.txt")
TYPES = ["spatial", "temporal", "cross"]


def _load():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            kv = dict(t.split("=") for t in tok[2:])
            cur = {"name": tok[1], "N": int(kv["N"]), "lo": int(kv["lo"]), "hi": int(kv["hi"]),
                   "cand": [int(x) for x in kv["candidates"].split(",")], "diff": {},
                   "blocks": int(kv.get("blocks", "1"))}
            cases.append(cur)
        elif tok[0] == "diff":
            # "diff <type>" (block 0) or "diff <type>/<block>"
            name, _, blk = tok[1].partition("/")
            cur["diff"][(name, int(blk or 0))] = [float(x) for x in tok[2:]]
        elif tok[0] == "expect":
            if tok[1] == "error":
                cur["error"] = True
            else:
                kv = dict(t.split("=") for t in tok[1:])
                cur["ranges"] = [int(x) for x in kv["ranges"].split(",")]
                cur["scores"] = [float(x) for x in kv["scores"].split(",")]
    return cases


def _matrix(case, block=0):
    names = [t for t in TYPES if (t, block) in case["diff"]]
    return [[case["diff"][(t, block)][i] for t in names] for i in range(case["N"])]


def _stack(case):
    return [_matrix(case, b) for b in range(case["blocks"])]


@pytest.mark.parametrize("case", _load(), ids=lambda c: c["name"])
def test_oracle_hand_cases(case):
    assert all(len(v) == case["N"] for v in case["diff"].values())
    assert len({k[1] for k in case["diff"]}) == case["blocks"]
    fn = (lambda: oracle.calibrate_ranges(_matrix(case), case["cand"], case["lo"], case["hi"])) \
        if case["blocks"] == 1 else \
        (lambda: oracle.calibrate_ranges_stack(_stack(case), case["cand"], case["lo"], case["hi"]))
    if case.get("error"):
        with pytest.raises(ValueError):
            fn()
        return
    ranges, scores = fn()
    assert ranges == case["ranges"]
    assert scores == case["scores"]


def test_stack_of_one_is_single_block():
    for case in _load():
        if case["blocks"] == 1 and not case.get("error"):
            assert oracle.calibrate_ranges_stack([_matrix(case)], case["cand"], case["lo"],
                                                 case["hi"]) == \
                oracle.calibrate_ranges(_matrix(case), case["cand"], case["lo"], case["hi"])


def test_stack_of_identical_blocks_is_one_block():
    # The mean over blocks of identical differences is the one block's mean
    # (exactly, for these dyadic values).
    rng = np.random.default_rng(3)
    diff = (rng.integers(0, 64, (30, 3)) / 64.0).tolist()
    one = oracle.calibrate_ranges(diff, [2, 4, 6])
    assert oracle.calibrate_ranges_stack([diff] * 4, [2, 4, 6]) == one


def test_stack_score_is_mean_of_block_scores():
    # Reading of the stack: a type's score is its mean difference over every
    # block and counted step, i.e. the mean of the blocks' own scores (equal
    # counts per block).  Dyadic values keep every sum exact; the division
    # by the 20 counted steps rounds, so the two orders agree to an ulp.
    rng = np.random.default_rng(11)
    blocks = [(rng.integers(0, 256, (30, 3)) / 256.0).tolist() for _ in range(5)]
    per_block = [oracle.calibrate_ranges(b, [2, 4, 6])[1] for b in blocks]
    _, scores = oracle.calibrate_ranges_stack(blocks, [2, 4, 6])
    for a in range(3):
        assert math.isclose(scores[a], sum(pb[a] for pb in per_block) / len(blocks),
                            rel_tol=1e-15, abs_tol=0.0)


def test_stack_block_order_does_not_matter():
    rng = np.random.default_rng(12)
    blocks = [(rng.integers(0, 256, (30, 3)) / 256.0).tolist() for _ in range(6)]
    want = oracle.calibrate_ranges_stack(blocks, [1, 3, 5])
    for perm in ([5, 4, 3, 2, 1, 0], [2, 0, 4, 1, 5, 3]):
        assert oracle.calibrate_ranges_stack([blocks[i] for i in perm], [1, 3, 5]) == want


def c_calibrate(diff, cand, lo=15, hi=85):
    d = np.ascontiguousarray(np.asarray(diff, dtype=np.float64))
    if d.ndim == 2:
        d = d[None]
    nb, n, t = d.shape
    c = np.ascontiguousarray(np.asarray(cand, dtype=np.int32))
    out = np.zeros(t, dtype=np.int32)
    sc = np.zeros(t, dtype=np.float64)
    st = lib.load().pab_plan_calibrate(
        nb, n, t, d.ctypes.data_as(C.POINTER(C.c_double)), lo, hi,
        c.ctypes.data_as(C.POINTER(C.c_int32)), out.ctypes.data_as(C.POINTER(C.c_int32)),
        sc.ctypes.data_as(C.POINTER(C.c_double)))
    return st, out.tolist(), sc.tolist()


@pytest.mark.parametrize("case", _load(), ids=lambda c: c["name"])
def test_c_planner_hand_cases(case):
    st, ranges, scores = c_calibrate(_stack(case), case["cand"], case["lo"], case["hi"])
    if case.get("error"):
        assert st == lib.PAB_ERR_INVALID_ARG
        return
    assert st == lib.PAB_OK
    assert ranges == case["ranges"] and scores == case["scores"]


def test_c_matches_oracle_random():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(3, 60))
        t = int(rng.integers(1, 6))
        lo = int(rng.integers(0, 40))
        hi = int(rng.integers(lo, 101))
        diff = rng.random((n, t)) * (10.0 ** rng.integers(-8, 3))
        if trial % 5 == 0:  # force ties
            diff[:, -1] = diff[:, 0]
        cand = rng.integers(0, 9, size=t).tolist()
        try:
            want = oracle.calibrate_ranges(diff.tolist(), cand, lo, hi)
        except ValueError:
            st, _, _ = c_calibrate(diff, cand, lo, hi)
            assert st == lib.PAB_ERR_INVALID_ARG
            continue
        st, ranges, scores = c_calibrate(diff, cand, lo, hi)
        assert st == lib.PAB_OK
        assert ranges == want[0]
        assert scores == want[1]


def test_invariances():
    rng = np.random.default_rng(5)
    n, t = 30, 3
    diff = rng.random((n, t))
    cand = [2, 4, 6]
    base, _ = oracle.calibrate_ranges(diff.tolist(), cand)
    # Scaling by a power of two keeps every comparison.
    assert oracle.calibrate_ranges((diff * 2.0 ** -20).tolist(), cand)[0] == base
    # Relabelling the types relabels the ranges.
    perm = [2, 0, 1]
    got, _ = oracle.calibrate_ranges(diff[:, perm].tolist(), cand)
    assert got == [base[p] for p in perm]
    # Steps outside the window (and the window's first step) never count.
    d2 = diff.copy()
    for i in range(n):
        if not (oracle.in_window(i, n) and oracle.in_window(i - 1, n)):
            d2[i] = rng.random(t) * 1e6
    assert oracle.calibrate_ranges(d2.tolist(), cand)[0] == base
    # Smaller change -> wider range (the pyramid the pages describe).
    ranges, scores = oracle.calibrate_ranges(diff.tolist(), cand)
    for a in range(t):
        for b in range(t):
            if scores[a] > scores[b]:
                assert ranges[a] <= ranges[b]


def test_c_validation():
    L = lib.load()
    d = np.ones((10, 3))
    assert c_calibrate(d, [2, -1, 3])[0] == lib.PAB_ERR_INVALID_ARG
    bad = d.copy()
    bad[5, 1] = np.nan
    assert c_calibrate(bad, [2, 4, 6])[0] == lib.PAB_ERR_INVALID_ARG
    bad[5, 1] = -1.0
    assert c_calibrate(bad, [2, 4, 6])[0] == lib.PAB_ERR_INVALID_ARG
    bad[5, 1] = np.inf
    assert c_calibrate(bad, [2, 4, 6])[0] == lib.PAB_ERR_INVALID_ARG
    # Outside the window anything goes: it is never read.
    ok = d.copy()
    ok[0, 0] = np.nan
    assert c_calibrate(ok, [2, 4, 6])[0] == lib.PAB_OK
    assert c_calibrate(d, [2, 4, 6], lo=50, hi=40)[0] == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_calibrate(1, 10, 3, None, 15, 85, None, None, None) == lib.PAB_ERR_INVALID_ARG
    # No blocks; a bad value in the second block's window.
    dd = np.ascontiguousarray(np.ones((2, 10, 3)))
    c = np.ascontiguousarray(np.array([2, 4, 6], dtype=np.int32))
    out = np.zeros(3, dtype=np.int32)
    args = (dd.ctypes.data_as(C.POINTER(C.c_double)), 15, 85,
            c.ctypes.data_as(C.POINTER(C.c_int32)), out.ctypes.data_as(C.POINTER(C.c_int32)), None)
    assert L.pab_plan_calibrate(0, 10, 3, *args) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_calibrate(2, 10, 3, *args) == lib.PAB_OK
    dd[1, 4, 2] = np.nan
    assert L.pab_plan_calibrate(2, 10, 3, *args) == lib.PAB_ERR_INVALID_ARG
    assert "block 1" in lib.pab_last_error()
    assert L.pab_plan_calibrate(1, 10, 3, *args) == lib.PAB_OK  # block 1 not read


def test_c_matches_oracle_random_stacks():
    rng = np.random.default_rng(12)
    for trial in range(100):
        nb = int(rng.integers(1, 5))
        n = int(rng.integers(3, 40))
        t = int(rng.integers(1, 5))
        diff = rng.random((nb, n, t)) * (10.0 ** rng.integers(-8, 3))
        cand = rng.integers(0, 9, size=t).tolist()
        want = oracle.calibrate_ranges_stack(diff.tolist(), cand)
        st, ranges, scores = c_calibrate(diff, cand)
        assert st == lib.PAB_OK
        assert ranges == want[0] and scores == want[1]
