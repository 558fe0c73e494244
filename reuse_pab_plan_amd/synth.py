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
* ``gpu_tensor`` -- the library's device generator (``pab_synth_normal``,
  declared in ``include/pab_synth.h``): Philox4x32-10 streams (Salmon,
  Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC'11) keyed by the stream number below, turned into normals by the
  Box-Muller transform.  torch only provides the device memory.  Every
  tensor is regenerated from its counters on demand, so no base tensor is
  stored.

The two are *not* bitwise equal to each other; each is deterministic given
its seed.  ``philox4x32_10`` and ``philox_normals`` restate the device
generator's definition on the host (numpy), so its raw words can be checked
bit for bit and its normals to fp32 rounding.
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


def _synth_normal(out, key_a, scale_a, key_b=0, scale_b=0.0, stream=None):
    """out[e] = round(scale_a * N(key_a)[e] + scale_b * N(key_b)[e]) on the
    device (the library's Philox4x32-10 + Box-Muller generator)."""
    from . import lib

    return lib.pab_synth_normal(out, key_a, scale_a, key_b, scale_b, stream=stream)


def gpu_tensor(shape, config_seed, block, type_idx, tensor, step, n_steps, dtype="bf16",
               device="cuda", out=None, perturb=True, stream=None):
    """One perturbed input tensor generated on the device.

    ``base + sigma_step * eps`` with base and eps each a Philox4x32-10 normal
    stream (keys: the stream numbers of the base and of the step), formed in
    fp32 and rounded once to the dtype.  If ``out`` is given the result is
    written into it (same number of elements and dtype; contiguous).  With
    ``perturb=False`` the base tensor alone is returned (the same at every
    step).
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty(shape, dtype=tdt, device=device)
    key_base = stream_id(config_seed, block, type_idx, tensor, -1)
    if perturb:
        key_eps = stream_id(config_seed, block, type_idx, tensor, step)
        _synth_normal(out, key_base, 1.0, key_eps, step_sigma(step, n_steps), stream)
    else:
        _synth_normal(out, key_base, 1.0, 0, 0.0, stream)
    return out


WEIGHTS = {"w_in": 0, "w_kv": 1, "w_out": 2}


def gpu_weight(shape, config_seed, block, type_idx, which, dtype="bf16", device="cuda",
               stream=None):
    """A fixed projection weight [out, in] ~ N(0, 1/in), drawn on the device
    (the same at every step); ``which`` indexes ``WEIGHTS``."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = torch.empty(shape, dtype=tdt, device=device)
    key = stream_id(config_seed, block, type_idx, 8 + which, -1)
    return _synth_normal(w, key, float(shape[1]) ** -0.5, 0, 0.0, stream)


# ------------------------------------------------- host restatement (numpy)

PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers of Philox4x32
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key increments between rounds
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 on the host.

    counter: uint32 array [..., 4] (words c0..c3); key: uint32 array [..., 2]
    or a pair (k0, k1), broadcast against the counters.  Returns uint32
    [..., 4].  Each round multiplies c0 and c2 by the two round constants
    (64-bit products), XORs the high halves with the other two words and the
    key, and the key advances by the Weyl increments between rounds.
    """
    c = np.asarray(counter, dtype=np.uint64)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint64), c.shape[:-1] + (2,))
    c0, c1, c2, c3 = (c[..., j].copy() for j in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for _ in range(10):
        p0 = m0 * c0          # < 2^64: exact in uint64
        p1 = m1 * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ k0
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ k1
        c1 = p1 & _U32
        c3 = p0 & _U32
        c0, c2 = n0, n2
        k0 = (k0 + np.uint64(PHILOX_W[0])) & _U32
        k1 = (k1 + np.uint64(PHILOX_W[1])) & _U32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def philox_blocks(key: int, block0: int, nblocks: int):
    """Blocks block0 .. block0+nblocks-1 of stream ``key``: uint32 [nblocks, 4]
    (counter (lo32(i), hi32(i), 0, 0), key (lo32(key), hi32(key)))."""
    i = np.arange(block0, block0 + nblocks, dtype=np.uint64)
    ctr = np.zeros((nblocks, 4), dtype=np.uint64)
    ctr[:, 0] = i & _U32
    ctr[:, 1] = i >> np.uint64(32)
    return philox4x32_10(ctr, (key & 0xFFFFFFFF, key >> 32))


def philox_normals(key: int, n: int):
    """The first n standard normals of stream ``key`` (float64 Box-Muller of
    the exact Philox words; the device forms the same in fp32)."""
    w = philox_blocks(key, 0, (n + 3) // 4).astype(np.float64)
    u = (np.floor(w[:, 0::2] / 512.0) + 0.5) * 2.0 ** -23
    v = (np.floor(w[:, 1::2] / 512.0) + 0.5) * 2.0 ** -23
    r = np.sqrt(-2.0 * np.log(u))
    z = np.empty((w.shape[0], 4))
    z[:, 0::2] = r * np.cos(2 * np.pi * v)
    z[:, 1::2] = r * np.sin(2 * np.pi * v)
    return z.reshape(-1)[:n]
