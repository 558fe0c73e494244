"""Pins of the projection oracle (block context around the attention).

Identity weights must move every input feature to the head/channel the
layout reading names; small integer inputs give exact products; torch's CPU
fp64 linear agrees; relabelling heads in the weight relabels the outputs;
and a round trip (input projection with identity weights, output projection
with identity weights) returns the input.
"""

import numpy as np
import torch

import oracle

rng = np.random.default_rng(3)


def test_identity_weight_places_features():
    B, F, S, H, D = 2, 3, 5, 4, 8
    C = H * D
    x = rng.standard_normal((B, F * S, C))
    w = np.concatenate([np.eye(C)] * 3)            # q = k = v = x
    q, k, v = oracle.proj_in(x, w, H, D, F, S)
    for t in (q, k, v):
        assert t.shape == (B, H, F, S, D)
        for b in range(B):
            for f in range(F):
                for s in range(S):
                    for h in range(H):
                        assert np.array_equal(t[b, h, f, s], x[b, f * S + s, h * D:(h + 1) * D])


def test_round_trip_identity():
    B, F, S, H, D = 1, 2, 7, 3, 16
    C = H * D
    x = rng.standard_normal((B, F * S, C))
    (q,) = oracle.proj_in(x, np.eye(C), H, D, F, S)
    assert np.array_equal(oracle.proj_out(q, np.eye(C)), x)


def test_exact_small_integers():
    B, F, S, H, D = 1, 1, 4, 2, 4
    C = H * D
    x = rng.integers(-3, 4, size=(B, F * S, C)).astype(np.float64)
    w = rng.integers(-2, 3, size=(2 * C, C)).astype(np.float64)
    k, v = oracle.proj_in(x, w, H, D, F, S)
    # Hand check of one element: k[0, 1, 0, 2, 3] = x[0, 2, :] . w[1*D + 3, :]
    assert k[0, 1, 0, 2, 3] == float(np.dot(x[0, 2], w[1 * D + 3]))
    assert v[0, 0, 0, 1, 2] == float(np.dot(x[0, 1], w[C + 0 * D + 2]))


def test_matches_torch_linear():
    B, F, S, H, D = 2, 2, 9, 3, 8
    C = H * D
    x = rng.standard_normal((B, F * S, C))
    w = rng.standard_normal((3 * C, C))
    y = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    q, k, v = oracle.proj_in(x, w, H, D, F, S)
    assert np.max(np.abs(q.transpose(0, 2, 3, 1, 4).reshape(B, F * S, C) - y[..., :C])) <= 1e-12
    assert np.max(np.abs(v.transpose(0, 2, 3, 1, 4).reshape(B, F * S, C) - y[..., 2 * C:])) <= 1e-12
    o = rng.standard_normal((B, H, F, S, D))
    wo = rng.standard_normal((C, C))
    yo = torch.nn.functional.linear(
        torch.from_numpy(o.transpose(0, 2, 3, 1, 4).reshape(B, F * S, C).copy()), torch.from_numpy(wo)).numpy()
    assert np.max(np.abs(oracle.proj_out(o, wo) - yo)) <= 1e-12


def test_head_relabelling():
    B, F, S, H, D = 1, 1, 6, 3, 4
    C = H * D
    x = rng.standard_normal((B, F * S, C))
    w = rng.standard_normal((C, C))
    perm = [2, 0, 1]
    wp = np.concatenate([w[p * D:(p + 1) * D] for p in perm])
    (q,) = oracle.proj_in(x, w, H, D, F, S)
    (qp,) = oracle.proj_in(x, wp, H, D, F, S)
    for h, p in enumerate(perm):
        assert np.array_equal(qp[0, h], q[0, p])


def test_module_identity_projections_is_attention():
    # With identity projections the module is the attention itself (its
    # output read token-major).
    B, F, S, H, D = 1, 2, 5, 2, 8
    C = H * D
    x = rng.standard_normal((B, F * S, C))
    eye3 = np.concatenate([np.eye(C)] * 3)
    for kind, fn in (("spatial", oracle.spatial), ("temporal", oracle.temporal)):
        got = oracle.module(kind, x, eye3, np.eye(C), H, D, F, S)
        (q,) = oracle.proj_in(x, np.eye(C), H, D, F, S)
        want = oracle.proj_out(fn(q, q, q), np.eye(C))
        assert np.max(np.abs(got - want)) <= 1e-12
    xt = rng.standard_normal((B, 3, C))
    got = oracle.module("cross", x, np.eye(C), np.eye(C), H, D, F, S, x_text=xt,
                        w_kv=np.concatenate([np.eye(C)] * 2), text_len=[2])
    (q,) = oracle.proj_in(x, np.eye(C), H, D, F, S)
    (kt,) = oracle.proj_in(xt, np.eye(C), H, D, 1, 3)
    want = oracle.proj_out(oracle.cross(q, kt[:, :, 0], kt[:, :, 0], text_len=[2]), np.eye(C))
    assert np.max(np.abs(got - want)) <= 1e-12
