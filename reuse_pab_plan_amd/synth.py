"""Seeded synthetic inputs for the PAB attention path.

This module holds no arithmetic of the method: it only draws the Q, K, V
tensors a video DiT block would hand to its attentions, so that the tests,
the benchmark and the oracle all see the same bytes.

Workload recipe (stand-in for the trained models' features, which are not
available): per (config seed, block, attention type, tensor) a base tensor
``base ~ N(0, 1)``; at denoising step ``i`` the tensor is

    X_i = base + sigma_i * eps_i,   eps_i ~ N(0, 1) fresh per step,

with ``sigma_i = 0.5`` in the first and last 15% of the steps and ``0.02`` in
between, which gives consecutive-step differences the U shape the PAB article
reports ("Implementation", first observation).  Values are drawn in fp32 and
rounded to the working dtype (bf16 rounds to nearest even).

Attention-module workloads draw the module input instead: token-major
``x`` [B, F*S, C] (and the text tokens [B, L, C] of a cross attention)
follow the same perturbation model, and each projection weight is a fixed
``N(0, 1/C)`` matrix per (block, type), so that projected Q/K/V have unit
variance like the attention-only inputs.

Two generators draw the same distribution:

* ``cpu_tensor`` -- numpy PCG64 streams, for small shapes and CPU tests;
* ``gpu_tensor`` -- torch's device Philox generator, for full-size shapes that
  live in HBM.  The two are *not* bitwise equal to each other; each is
  deterministic given its seed.
"""

from __future__ import annotations

import numpy as np

TENSORS = {"q": 0, "k": 1, "v": 2}
OUTER_SIGMA = 0.5
INNER_SIGMA = 0.02


def step_sigma(step: int, n_steps: int) -> float:
    """Perturbation scale of the workload at ``step``: large on the outer 15%
    of the steps at either end, small in between (integer test on step/N)."""
    outer = 100 * step < 15 * n_steps or 100 * step >= 85 * n_steps
    return OUTER_SIGMA if outer else INNER_SIGMA


def stream_id(config_seed: int, block: int, type_idx: int, tensor: int, step: int) -> int:
    """Injective 63-bit stream number; ``step = -1`` names the base tensor."""
    if not (0 <= block < 4096 and 0 <= type_idx < 16 and 0 <= tensor < 16 and -1 <= step < 65535):
        raise ValueError("stream_id: index out of range")
    return ((((config_seed * 4096 + block) * 16 + type_idx) * 16 + tensor) * 65536) + (step + 1)


def _np_normal(seed: int, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=shape, dtype=np.float32)


def cpu_tensor(shape, config_seed, block, type_idx, tensor, step, n_steps, dtype="f32"):
    """One perturbed input tensor on the host.

    Returns a torch CPU tensor of dtype float32 or bfloat16.
    """
    import torch

    base = _np_normal(stream_id(config_seed, block, type_idx, tensor, -1), shape)
    eps = _np_normal(stream_id(config_seed, block, type_idx, tensor, step), shape)
    x = torch.from_numpy(base + np.float32(step_sigma(step, n_steps)) * eps)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def gpu_tensor(shape, config_seed, block, type_idx, tensor, step, n_steps, dtype="bf16",
               device="cuda", out=None, perturb=True):
    """One perturbed input tensor generated on the device (torch Philox).

    If ``out`` is given the result is written into it (same shape and dtype).
    With ``perturb=False`` the base tensor alone is returned (the same at
    every step).
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(stream_id(config_seed, block, type_idx, tensor, -1))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if perturb:
        g.manual_seed(stream_id(config_seed, block, type_idx, tensor, step))
        eps = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.add_(eps, alpha=step_sigma(step, n_steps))
        del eps
    if out is None:
        return x.to(tdt)
    out.copy_(x)
    return out


WEIGHTS = {"w_in": 0, "w_kv": 1, "w_out": 2}


def gpu_weight(shape, config_seed, block, type_idx, which, dtype="bf16", device="cuda"):
    """A fixed projection weight [out, in] ~ N(0, 1/in), drawn on the device
    (the same at every step); ``which`` indexes ``WEIGHTS``."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(stream_id(config_seed, block, type_idx, 8 + which, -1))
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    w.mul_(float(shape[1]) ** -0.5)
    return w.to(tdt)
