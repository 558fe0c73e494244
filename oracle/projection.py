"""Projections around an attention: the block context of the PAB hot path.

What the pages fix (restated): the PAB article ("Implementation") broadcasts
the result of an attention computation to the following steps so that those
steps skip the attention computation; in a DiT block an attention is the
query/key/value projection of the block's input, the attention itself, and
the output projection (the features the article calls x_t pass through
them).  Skipping the attention on a broadcast step therefore skips both
projections with it: the cached quantity is the attention module's output.

Readings where the pages are open:

19. Weights use the layout of a linear layer, ``w[out_features, in_features]``
    with ``y = x @ w.T``, no bias.  Hidden size C = H * D; the input
    projection's outputs are grouped per tensor then per head: output feature
    ``j`` of the q/k/v projection is tensor ``j // C``, head ``(j % C) // D``,
    channel ``j % D``.
20. Token order: a video entry's F*S tokens are frame-major (token
    ``f*S + s``), the same order as the attention layout [B, H, F, S, D].

Everything in fp64 after exact widening of the inputs.
"""

from __future__ import annotations

import numpy as np

from .attention import _wide


def linear(x, w):
    """y = x @ w.T in fp64 (x [..., in], w [out, in])."""
    return _wide(x) @ _wide(w).T


def proj_in(x, w, n_heads: int, head_dim: int, frames: int, tokens: int):
    """Input projection to head-major tensors.

    x: [B, F*S, C] (C = H*D); w: [n*C, C] with n the number of output tensors
    (3 for q, k, v; 2 for k, v of the text; 1 for q).  Returns a list of n
    arrays [B, H, F, S, D].
    """
    x = _wide(x)
    b, t, c = x.shape
    if c != n_heads * head_dim or t != frames * tokens:
        raise ValueError("shape mismatch")
    y = linear(x, w)                                       # [B, T, n*C]
    n = y.shape[-1] // c
    y = y.reshape(b, frames, tokens, n, n_heads, head_dim)  # token f*S+s, feature (i, h, d)
    return [np.ascontiguousarray(y[:, :, :, i].transpose(0, 3, 1, 2, 4)) for i in range(n)]


def proj_out(o, w):
    """Output projection of a head-major attention output.

    o: [B, H, F, S, D]; w: [C, C].  Returns y [B, F*S, C] with the input
    feature of (h, d) at index h*D + d.
    """
    o = _wide(o)
    b, h, f, s, d = o.shape
    tokens = o.transpose(0, 2, 3, 1, 4).reshape(b, f * s, h * d)
    return linear(tokens, w)


def module(kind: str, x, w_in, w_out, n_heads: int, head_dim: int, frames: int, tokens: int,
           x_text=None, w_kv=None, text_len=None, scale=None):
    """One attention module: input projection, attention, output projection.

    kind: "spatial" / "temporal" / "cross".  x: [B, F*S, C]; w_in: [3C, C]
    (cross: [C, C], the query projection, with w_kv [2C, C] projecting the
    text tokens x_text [B, L, C]); w_out: [C, C].  Returns [B, F*S, C].
    """
    from . import attention as _attn

    if kind == "cross":
        (q,) = proj_in(x, w_in, n_heads, head_dim, frames, tokens)
        xt = _wide(x_text)
        k, v = proj_in(xt, w_kv, n_heads, head_dim, 1, xt.shape[1])
        o = _attn.cross(q, k[:, :, 0], v[:, :, 0], scale, text_len=text_len)
    else:
        q, k, v = proj_in(x, w_in, n_heads, head_dim, frames, tokens)
        fn = _attn.spatial if kind == "spatial" else _attn.temporal
        o = fn(q, k, v, scale)
    return proj_out(o, w_out)
