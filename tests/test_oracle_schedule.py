"""Pins for oracle.schedule against facts fixed outside the oracle.

* hand-derived tables (tests/golden/schedule_tables.txt);
* the page-fixed split: 15% / 70% / 15% of the steps (PAB article,
  "Implementation", first observation);
* closed-form counts, r = 0 is PAB off, the pyramid ordering (wider range,
  fewer recomputes: PAB article, Figure 2 caption), and that every reuse
  draws on a computed in-window step no more than r steps earlier.
"""

import os

import numpy as np
import pytest

from oracle import closed_form_counts, in_window, schedule, window_bounds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_tables.txt")


def _load_golden():
    cases, cur = [], None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "case":
                n = int(parts[2].split("=")[1])
                ranges = [int(x) for x in parts[3].split("=")[1].split(",")]
                cur = {"name": parts[1], "n": n, "ranges": ranges, "rows": []}
                cases.append(cur)
            else:
                entries = parts[1:-1]
                count = int(parts[-1].split("=")[1])
                cur["rows"].append((parts[0], entries, count))
    return cases


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_hand_derived_tables(case):
    rec, src, cnt = schedule(case["n"], case["ranges"])
    for a, (_, entries, count) in enumerate(case["rows"]):
        assert len(entries) == case["n"]
        for i, e in enumerate(entries):
            if e == "X":
                assert rec[i, a] == 1 and src[i, a] == i
            else:
                assert rec[i, a] == 0 and src[i, a] == int(e)
        assert cnt[a] == count


@pytest.mark.parametrize("n", [10, 20, 30, 50, 100])
def test_seventy_percent_middle(n):
    # 15% + 70% + 15%: for these N, 0.15*N, 0.7*N are whole or half steps;
    # the half-open integer test keeps exactly 70% inside.
    w0, w = window_bounds(n)
    assert w * 10 == n * 7
    assert sum(in_window(i, n) for i in range(n)) == w
    inside = [i for i in range(n) if in_window(i, n)]
    assert inside == list(range(w0, w0 + w))  # contiguous
    # first 15% rounded up, last 15% rounded down
    assert w0 == -(-15 * n // 100)


def test_window_edges_exact():
    assert [in_window(i, 30) for i in (4, 5, 25, 26)] == [False, True, True, False]
    assert window_bounds(10) == (2, 7)
    assert window_bounds(30) == (5, 21)
    assert window_bounds(50) == (8, 35)


@pytest.mark.parametrize("n", list(range(1, 61)) + [97, 200])
@pytest.mark.parametrize("r", [0, 1, 2, 3, 4, 5, 6, 9, 12])
@pytest.mark.parametrize("win", [(15, 85), (0, 100), (50, 50), (0, 0), (30, 60)])
def test_closed_form_and_properties(n, r, win):
    lo, hi = win
    rec, src, cnt = schedule(n, [r], lo, hi)
    assert cnt[0] == closed_form_counts(n, [r], lo, hi)[0]
    assert cnt[0] == rec[:, 0].sum()
    for i in range(n):
        j = src[i, 0]
        if rec[i, 0]:
            assert j == i
        else:
            # reuse: source computed, in the window, at most r steps back,
            # and every step between source and i is a reuse in the window
            assert rec[j, 0] == 1 and j < i <= j + r
            assert in_window(j, n, lo, hi) and in_window(i, n, lo, hi)
            assert all(rec[t, 0] == 0 and in_window(t, n, lo, hi) for t in range(j + 1, i + 1))
        if not in_window(i, n, lo, hi):
            assert rec[i, 0] == 1
    if r == 0:
        assert cnt[0] == n  # PAB off recomputes every step
    if n >= 1:
        assert rec[0, 0] == 1  # the first step always computes


def test_pyramid_ordering():
    # spatial < temporal < cross ranges -> non-increasing recompute counts
    for n in range(1, 80):
        _, _, cnt = schedule(n, [2, 4, 6])
        assert cnt[0] >= cnt[1] >= cnt[2]
        _, _, cnt = schedule(n, [0, 1, 2, 3, 7])
        assert all(cnt[a] >= cnt[a + 1] for a in range(4))


def test_brute_force_enumeration():
    # Independent statement: inside the window, step i computes iff
    # (i - first_window_step) is a multiple of (r + 1).
    for n in range(1, 70):
        w0, _ = window_bounds(n)
        for r in range(0, 8):
            rec, _, _ = schedule(n, [r])
            for i in range(n):
                expect = (not in_window(i, n)) or ((i - w0) % (r + 1) == 0)
                assert rec[i, 0] == int(expect)


def test_bad_arguments():
    with pytest.raises(ValueError):
        schedule(0, [1])
    with pytest.raises(ValueError):
        schedule(10, [-1])
    with pytest.raises(ValueError):
        schedule(10, [1], 60, 40)


def test_types_independent():
    rec, src, _ = schedule(30, [2, 4, 6])
    for a, r in enumerate([2, 4, 6]):
        r1, s1, _ = schedule(30, [r])
        assert np.array_equal(rec[:, a], r1[:, 0]) and np.array_equal(src[:, a], s1[:, 0])

