"""CPU oracle for the Pyramid Attention Broadcast (PAB) attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, constant or helper with the HIP
library under ``reuse_pab_plan_amd/``; it imports numpy and the standard
library only.  All floating point is fp64, after exact widening of the
caller's inputs (bf16 and fp32 both widen to fp64 without rounding).

Sources (two web pages describing the method; the oracle cites them by name):

* "PAB article" -- the English page *The first real-time AI video generation
  technology in history: DiT universal, 10.6 times faster* (php.cn), with its
  sections "pyramid attention broadcast", "Implementation", "Parallel" and
  its Figure 1 / Figure 2 captions.
* "PAB abstract" -- *Real-Time Video Generation with Pyramid Attention
  Broadcast* (Zhao, Jin, Wang, You, 2024), Abstract.

Modules:

* ``schedule``   -- which (step, attention type) pairs recompute and which
                    step each reuse takes its output from (pinned: closed-form
                    counts, brute-force properties, hand-derived tables), and
                    the per-type ranges calibrated from a measured attention
                    difference (pinned: hand-derived cases, invariances).
* ``attention``  -- softmax(Q K^T * scale) V written out plainly, and the three
                    gathers of it (spatial, temporal, cross) (pinned: row sums,
                    permutation invariance, single key, Q = 0, closed-form
                    two-key case, literal loops, torch CPU fp64 SDPA).
* ``mse``        -- mean squared difference of two attention outputs (pinned:
                    hand example, identities, exact dyadic shifts).
* ``projection`` -- the input (q/k/v) and output projections around an
                    attention, in head-major layout (pinned: identity
                    weights, exact small integers, torch CPU fp64 linear,
                    head relabelling).
* ``trajectory`` -- the broadcast cache run over a whole denoising trajectory
                    (pinned: PAB-off equals per-step attention, reuse is
                    identity, recompute count equals the closed form).
"""

from .schedule import (  # noqa: F401
    in_window,
    window_bounds,
    schedule,
    closed_form_counts,
    calibrate_ranges,
    calibrate_ranges_stack,
)
from .attention import (  # noqa: F401
    attn_loop,
    attn_fp64,
    softmax_rows,
    spatial,
    temporal,
    cross,
    spatial_rows,
    temporal_positions,
    cross_rows,
)
from .mse import mse  # noqa: F401
from .projection import linear, proj_in, proj_out, module  # noqa: F401
from .trajectory import trajectory  # noqa: F401
