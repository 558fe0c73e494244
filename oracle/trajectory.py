"""The broadcast cache run over a whole denoising trajectory.

PAB article, Figure 2 caption: at run time the attention result of a step is
broadcast to the next few steps so they skip the attention computation.  The
oracle runs that literally: for each step and attention type, either compute
the attention from that step's inputs and remember it, or hand back the
remembered output of the source step.  The schedule comes from
``oracle.schedule``.
"""

from __future__ import annotations

from . import attention as _attn
from .mse import mse as _mse
from .schedule import schedule as _schedule

_KERNELS = {
    "spatial": lambda x: _attn.spatial(x["q"], x["k"], x["v"], x.get("scale")),
    "temporal": lambda x: _attn.temporal(x["q"], x["k"], x["v"], x.get("scale")),
    "cross": lambda x: _attn.cross(x["q"], x["k"], x["v"], x.get("scale")),
}


def trajectory(n_steps, kinds, ranges, inputs_fn, lo_pct=15, hi_pct=85, compute=None):
    """Run the cache.

    Args:
      n_steps: N.
      kinds:   attention type names, one per type ("spatial"/"temporal"/"cross").
      ranges:  broadcast range per type.
      inputs_fn(step, type_index) -> dict with "q", "k", "v" (and optional
               "scale"); called only where the schedule recomputes.
      compute: optional function (kind, inputs) -> output replacing the
               attention (e.g. a whole attention module).

    Returns a dict with
      "outputs":   outputs[i][a], the attention output of step i, type a
                   (the same ndarray object as its source step when reused);
      "recompute", "source", "counts": the schedule;
      "drift":     drift[i][a] = mse(output, previous recomputed output of the
                   same type) at recompute steps that have a predecessor,
                   else None (the attention difference of the Figure 1
                   caption, taken between successive computations).
      "calls":     number of attention evaluations performed.
    """
    recompute, source, counts = _schedule(n_steps, ranges, lo_pct, hi_pct)
    cache = [None] * len(kinds)
    outputs, drift = [], []
    calls = 0
    for i in range(n_steps):
        row, drow = [], []
        for a, kind in enumerate(kinds):
            if recompute[i, a]:
                x = inputs_fn(i, a)
                out = compute(kind, x) if compute is not None else _KERNELS[kind](x)
                calls += 1
                drow.append(None if cache[a] is None else _mse(out, cache[a]))
                cache[a] = out
            else:
                drow.append(None)
            row.append(cache[a])
        outputs.append(row)
        drift.append(drow)
    return {
        "outputs": outputs,
        "recompute": recompute,
        "source": source,
        "counts": counts,
        "drift": drift,
        "calls": calls,
    }
