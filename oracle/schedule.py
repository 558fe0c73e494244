"""Broadcast schedule of Pyramid Attention Broadcast, written out step by step.

What the pages fix (restated, not quoted):

* PAB article, "Implementation", first observation: the attention difference
  between consecutive diffusion steps is U-shaped -- large in the first and the
  last 15% of the steps, small in the middle 70%.  PAB abstract says the same
  (a U-shaped attention difference implies redundancy).
* PAB article, "Implementation", second paragraph, and Figure 2 caption:
  inside that stable middle, one step's attention output is broadcast to
  several following steps, so those steps skip the attention computation.
  Each attention type gets its own broadcast range; the smaller a type's
  change, the wider its range (spatial changes most, cross attention least).
  PAB abstract: the ranges form a "pyramid" set per type by its variance.

Readings taken where the pages are open:

1. ``r`` (the range) is the number of following steps that reuse one computed
   output; the recompute period inside the window is ``r + 1``.  ``r = 0`` is
   PAB off.
2. Step ``i`` (0-based, execution order, 0 = noisiest) is in the stable window
   iff ``i/N`` lies in the half-open interval ``[lo/100, hi/100)``, evaluated in
   integers (``100*i >= lo*N`` and ``100*i < hi*N``).  With lo = 15, hi = 85
   this puts exactly 70% of the steps in the window for N = 10, 30, 50.
3. The first in-window step computes; broadcasting starts from it.
4. Nothing is broadcast across the window's edges: a step outside the window
   always computes, and its output is never reused.

Everything here is integer arithmetic, so any correct implementation must
agree bit for bit.
"""

from __future__ import annotations

import numpy as np


def in_window(i: int, n_steps: int, lo_pct: int = 15, hi_pct: int = 85) -> bool:
    """True iff step ``i`` of ``n_steps`` lies in the stable middle window.

    PAB article, "Implementation", first observation (outer 15% of steps on
    each side change a lot, the middle 70% little); reading 2 above.
    """
    return 100 * i >= lo_pct * n_steps and 100 * i < hi_pct * n_steps


def window_bounds(n_steps: int, lo_pct: int = 15, hi_pct: int = 85):
    """(first in-window step, number of in-window steps) by enumeration.

    Returns (None, 0) when no step is in the window.
    """
    inside = [i for i in range(n_steps) if in_window(i, n_steps, lo_pct, hi_pct)]
    if not inside:
        return None, 0
    return inside[0], len(inside)


def schedule(n_steps: int, ranges, lo_pct: int = 15, hi_pct: int = 85):
    """Recompute flags, reuse sources and per-type recompute counts.

    Walks the steps in execution order, once per attention type, the way the
    PAB article's "Implementation" section and Figure 2 describe the method
    at run time: outside the stable window every step computes; inside it, a
    step that computes hands its output on to the next ``r`` steps, which
    compute nothing; the step after them computes again.

    Args:
      n_steps: number of denoising steps N (>= 1).
      ranges:  broadcast range r_a >= 0 per attention type a.
      lo_pct, hi_pct: window edges in percent of N (0 <= lo <= hi <= 100).

    Returns:
      recompute: uint8 [N, T], 1 where (step, type) computes attention.
      source:    int32 [N, T], the step whose output (step, type) uses
                 (itself when it recomputes).
      counts:    int32 [T], recomputes per type.
    """
    ranges = [int(r) for r in ranges]
    if n_steps < 1:
        raise ValueError("n_steps must be >= 1")
    if any(r < 0 for r in ranges):
        raise ValueError("ranges must be >= 0")
    if not (0 <= lo_pct <= hi_pct <= 100):
        raise ValueError("need 0 <= lo_pct <= hi_pct <= 100")
    n_types = len(ranges)
    recompute = np.zeros((n_steps, n_types), dtype=np.uint8)
    source = np.zeros((n_steps, n_types), dtype=np.int32)
    for a, r in enumerate(ranges):
        last_computed = None   # step whose output is being broadcast
        remaining = 0          # how many more steps may still reuse it
        for i in range(n_steps):
            if not in_window(i, n_steps, lo_pct, hi_pct):
                # Outer steps change a lot: always compute, never broadcast.
                recompute[i, a] = 1
                source[i, a] = i
                last_computed, remaining = None, 0
            elif remaining > 0:
                # Inside the window, within the broadcast range: reuse.
                recompute[i, a] = 0
                source[i, a] = last_computed
                remaining -= 1
            else:
                # Inside the window, range used up (or window just entered).
                recompute[i, a] = 1
                source[i, a] = i
                last_computed, remaining = i, r
    counts = recompute.sum(axis=0).astype(np.int32)
    return recompute, source, counts


def closed_form_counts(n_steps: int, ranges, lo_pct: int = 15, hi_pct: int = 85):
    """Recompute count per type in closed form: (N - W) + ceil(W / (r + 1)).

    W is the number of in-window steps.  Used as a pin for ``schedule``: the
    outer N - W steps all compute, and the window (a contiguous run of W
    steps) computes once every r + 1 steps starting at its first step.
    """
    _, w = window_bounds(n_steps, lo_pct, hi_pct)
    return np.array([(n_steps - w) + (w + r) // (r + 1) for r in ranges], dtype=np.int32)


def calibrate_ranges(diff, candidates, lo_pct: int = 15, hi_pct: int = 85):
    """Broadcast ranges per attention type from a measured attention difference.

    What the pages fix: the PAB article ("Implementation") sets each type's
    broadcast range from how much its attention output changes between
    consecutive steps in the stable middle -- the less a type changes, the
    wider its range -- and measures that change by the MSE between the
    outputs of consecutive steps (Figure 1 caption).  The PAB abstract calls
    the resulting set of ranges a pyramid chosen by each type's variance.

    Readings where the pages are open:

    5. The change of type a is scored by the plain mean of diff[i][a] over the
       steps i whose output and predecessor's output both lie in the stable
       window (i >= 1, in_window(i) and in_window(i - 1)); the sum runs in
       step order, in fp64.
    6. The ranges handed out are the caller's candidates, assigned by rank:
       the type with the largest score gets the smallest candidate, the next
       largest the next smallest, and so on.  Equal scores rank the lower
       type index as the larger one.

    Args:
      diff: [N][T] numbers; diff[i][a] is the MSE between type a's outputs at
            steps i and i-1 of a trajectory that computes every step (row 0
            is not used).
      candidates: T ranges (>= 0) to assign.
      lo_pct, hi_pct: window edges, as in ``schedule``.

    Returns:
      (ranges, scores): ranges[a] assigned to type a, and the score of each
      type (Python floats, i.e. fp64).
    """
    return calibrate_ranges_stack([diff], candidates, lo_pct, hi_pct)


def calibrate_ranges_stack(diffs, candidates, lo_pct: int = 15, hi_pct: int = 85):
    """``calibrate_ranges`` for a stack of blocks that share one schedule.

    Reading 7 (the pages calibrate a model, not a block): every block of a
    stack follows the same schedule, so a type's score is the mean of its
    counted differences over all blocks -- the sum runs block by block, each
    block's counted steps in step order, in fp64, and is divided by
    (blocks x counted steps).  One block is ``calibrate_ranges``.

    Args:
      diffs: [blocks][N][T] numbers, one ``calibrate_ranges`` matrix per block.
    """
    n_blocks = len(diffs)
    n_types = len(candidates)
    if n_blocks < 1 or n_types < 1:
        raise ValueError("need at least one block and one type")
    n_steps = len(diffs[0])
    if n_steps < 1 or any(len(d) != n_steps for d in diffs):
        raise ValueError("every block needs the same number (>= 1) of steps")
    if any(int(c) < 0 for c in candidates):
        raise ValueError("candidate ranges must be >= 0")
    if not (0 <= lo_pct <= hi_pct <= 100):
        raise ValueError("need 0 <= lo_pct <= hi_pct <= 100")
    counted = [i for i in range(1, n_steps)
               if in_window(i, n_steps, lo_pct, hi_pct) and in_window(i - 1, n_steps, lo_pct, hi_pct)]
    if not counted:
        raise ValueError("the window holds fewer than two consecutive steps")
    scores = []
    for a in range(n_types):
        total = 0.0
        for diff in diffs:
            for i in counted:
                d = float(diff[i][a])
                if not (d >= 0.0) or d == float("inf"):
                    raise ValueError("attention differences must be finite and >= 0")
                total += d
        scores.append(total / (len(counted) * n_blocks))
    # Most-changing type first; it receives the narrowest range.
    order = sorted(range(n_types), key=lambda a: (-scores[a], a))
    ascending = sorted(int(c) for c in candidates)
    ranges = [0] * n_types
    for rank, a in enumerate(order):
        ranges[a] = ascending[rank]
    return ranges, scores
