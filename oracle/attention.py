"""Attention written from its definition, in fp64, and its three gathers.

The quantity PAB computes and then reuses is an attention output (PAB
article, "pyramid attention broadcast" and Figure 2 caption; PAB abstract).
The pages do not print the attention formula; the oracle takes the standard
scaled dot-product attention of a transformer block:

    s_ij = scale * sum_d q_id k_jd          scale = 1/sqrt(D) by default
    p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
    o_id = sum_j p_ij v_jd

The full score row is materialised: no tiling, no running maximum, nothing
shared with the GPU kernels.  Subtracting the row maximum changes no value
mathematically; it only keeps exp() finite.

The three attention types of a video DiT block (PAB article,
"Implementation", second observation: spatial, temporal and cross/modal
attention) are the same operation over different token sets.  Video tensors
are head-major ``[B, H, F, S, D]`` (F frames, S tokens per frame); text K/V are
``[B, H, L, D]``:

* spatial  -- one sequence per (b, h, f): the S tokens of one frame;
* temporal -- one sequence per (b, h, s): the F frames at one token position;
* cross    -- per (b, h): all F*S video tokens query the L text tokens.
"""

from __future__ import annotations

import math

import numpy as np


def _wide(x):
    """Exact widening to fp64 (bf16/fp16/fp32 -> fp64 loses nothing)."""
    if hasattr(x, "detach"):  # a torch tensor handed in by a test
        import torch  # local: the oracle itself needs numpy only

        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(d: int) -> float:
    """1/sqrt(D), the usual softmax temperature of a transformer head."""
    return 1.0 / math.sqrt(d)


def attn_loop(q, k, v, scale=None):
    """One sequence, literal Python loops (tiny shapes only).

    q: [Lq, D], k: [Lk, D], v: [Lk, Dv].  Returns o: [Lq, Dv] (fp64 ndarray).
    """
    q, k, v = _wide(q), _wide(k), _wide(v)
    lq, d = q.shape
    lk = k.shape[0]
    dv = v.shape[1]
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((lq, dv), dtype=np.float64)
    for i in range(lq):
        scores = []
        for j in range(lk):
            acc = 0.0
            for t in range(d):
                acc += float(q[i, t]) * float(k[j, t])
            scores.append(scale * acc)
        top = max(scores)
        weights = [math.exp(s - top) for s in scores]
        total = math.fsum(weights)
        for t in range(dv):
            out[i, t] = math.fsum(weights[j] * float(v[j, t]) for j in range(lk)) / total
    return out


def softmax_rows(s):
    """Row-wise softmax of a score matrix (last axis), fp64."""
    s = _wide(s)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attn_fp64(q, k, v, scale=None):
    """Batched attention over the last two axes: [..., Lq, D] x [..., Lk, D].

    The score matrix is built whole with BLAS products; rows are normalised
    by the plain softmax above.
    """
    q, k, v = _wide(q), _wide(k), _wide(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    return np.matmul(softmax_rows(s), v)


# --------------------------------------------------------------------------
# The three gathers.  Each moves the attended axis next to D and calls the
# one definition above.
# --------------------------------------------------------------------------

def spatial(q, k, v, scale=None):
    """[B,H,F,S,D] -> [B,H,F,S,D]; attention among the S tokens of each frame."""
    return attn_fp64(q, k, v, scale)


def temporal(q, k, v, scale=None):
    """[B,H,F,S,D] -> [B,H,F,S,D]; attention among the F frames at each s."""
    q, k, v = _wide(q), _wide(k), _wide(v)
    t = lambda x: np.swapaxes(x, 2, 3)  # [B,H,S,F,D]
    return t(attn_fp64(t(q), t(k), t(v), scale))


def cross(q, k_text, v_text, scale=None, text_len=None):
    """Video queries against text keys/values.

    q: [B,H,F,S,D] or [B,H,Nq,D]; k_text, v_text: [B,H,L,D].
    text_len: optional per-batch number of real text tokens (1..L); the
    text tokens past it are padding and take no part (reading of a padded
    prompt: the video attends to the real tokens of its own prompt only).
    Returns an array shaped like q.
    """
    q = _wide(q)
    shape = q.shape
    qf = q.reshape(shape[0], shape[1], -1, shape[-1])
    if text_len is None:
        return attn_fp64(qf, k_text, v_text, scale).reshape(shape)
    if len(text_len) != shape[0]:
        raise ValueError("one text length per batch entry")
    out = np.empty(qf.shape, dtype=np.float64)
    for b, n in enumerate(text_len):
        n = int(n)
        if not 1 <= n <= k_text.shape[2]:
            raise ValueError("text lengths must lie in [1, L]")
        # Only the first n text tokens of entry b exist for its queries.
        out[b] = attn_fp64(qf[b], _wide(k_text[b])[:, :n], _wide(v_text[b])[:, :n], scale)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Sampled forms for full-size parity: only the requested outputs are formed,
# each from the complete key/value set of its own sequence.
# --------------------------------------------------------------------------

def spatial_rows(q, k, v, b, h, f, rows, scale=None):
    """Spatial output rows ``rows`` of frame (b, h, f): [len(rows), D]."""
    qq = _wide(q[b, h, f])[np.asarray(rows)]
    return attn_fp64(qq, k[b, h, f], v[b, h, f], scale)


def temporal_positions(q, k, v, b, h, positions, scale=None):
    """Temporal outputs at token positions ``positions`` of (b, h): [F, P, D]."""
    pos = np.asarray(positions)
    qq = np.swapaxes(_wide(q[b, h][:, pos]), 0, 1)  # [P, F, D]
    kk = np.swapaxes(_wide(k[b, h][:, pos]), 0, 1)
    vv = np.swapaxes(_wide(v[b, h][:, pos]), 0, 1)
    return np.swapaxes(attn_fp64(qq, kk, vv, scale), 0, 1)


def cross_rows(q_flat, k_text, v_text, b, h, rows, scale=None, n_text=None):
    """Cross output rows ``rows`` of (b, h); q_flat is [B,H,Nq,D].  With
    ``n_text``, only the first n_text text tokens take part."""
    qq = _wide(q_flat[b, h])[np.asarray(rows)]
    n = k_text.shape[2] if n_text is None else int(n_text)
    return attn_fp64(qq, _wide(k_text[b, h])[:n], _wide(v_text[b, h])[:n], scale)
