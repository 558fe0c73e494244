"""Pins for oracle.attention against facts that hold independently of it.

Each pin is chosen so that a plausible slip in the oracle fails it: a wrong
softmax axis (row sums, permutation), a wrong scale (closed-form two-key),
a transposed product (non-square closed form), a dropped max shift (large
logits), a wrong gather axis (locality pins and per-sequence loops), and the
whole thing against torch's CPU fp64 scaled_dot_product_attention.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (
    attn_fp64,
    attn_loop,
    cross,
    cross_rows,
    softmax_rows,
    spatial,
    spatial_rows,
    temporal,
    temporal_positions,
)

RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def test_rows_sum_to_one():
    s = rnd(5, 7, 33, scale=4.0)
    p = softmax_rows(s)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12


def test_permutation_invariance():
    q, k, v = rnd(9, 16), rnd(23, 16), rnd(23, 8)
    perm = RNG.permutation(23)
    o1 = attn_fp64(q, k, v)
    o2 = attn_fp64(q, k[perm], v[perm])
    assert np.max(np.abs(o1 - o2)) <= 1e-12


def test_single_key_returns_v_exactly():
    q, k, v = rnd(6, 8), rnd(1, 8), rnd(1, 8)
    assert np.array_equal(attn_fp64(q, k, v), np.repeat(v, 6, axis=0))
    assert np.array_equal(attn_loop(q, k, v), np.repeat(v, 6, axis=0))


def test_zero_query_gives_mean_of_v():
    k, v = rnd(11, 8), rnd(11, 5)
    o = attn_fp64(np.zeros((3, 8)), k, v)
    assert np.max(np.abs(o - v.mean(0))) <= 1e-14


def test_constant_v_rows():
    q, k = rnd(4, 8), rnd(13, 8)
    row = rnd(1, 6)
    o = attn_fp64(q, k, np.repeat(row, 13, axis=0))
    assert np.max(np.abs(o - row)) <= 1e-14


@pytest.mark.parametrize("x", [-3.0, 0.25, 2.0, 7.5])
def test_two_key_closed_form(x):
    # q = (x, 0, 0, 0), k1 = (1, 0, 0, 0), k2 = 0 -> logits (x/2, 0) with
    # D = 4, so weight of key 1 is the logistic function of x/2.
    d = 4
    q = np.zeros((1, d)); q[0, 0] = x
    k = np.zeros((2, d)); k[0, 0] = 1.0
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.0, 5.0, 2.0]])
    w = 1.0 / (1.0 + math.exp(-x / math.sqrt(d)))
    expect = w * v[0] + (1 - w) * v[1]
    assert np.max(np.abs(attn_fp64(q, k, v)[0] - expect)) <= 1e-14
    assert np.max(np.abs(attn_loop(q, k, v)[0] - expect)) <= 1e-14


def test_non_square_orientation():
    # 1 query, 3 keys with distinct logits: catches q/k swapped or v^T.
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.sqrt(2) * math.log(2), 0.0], [math.sqrt(2) * math.log(5), 0.0]])
    v = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0], [0.0, 0.0, 1.0]])
    # logits: 0, log 2, log 5 -> weights 1:2:5
    expect = np.array([[1.0, 2.0, 5.0]]) / 8.0
    assert np.max(np.abs(attn_fp64(q, k, v) - expect)) <= 1e-14


def test_large_logits_stay_finite():
    q = np.array([[1000.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 0.0]])
    v = np.array([[3.0], [-7.0]])
    o = attn_fp64(q, k, v)
    assert np.isfinite(o).all() and abs(o[0, 0] - 3.0) <= 1e-12


def test_loop_matches_vectorised():
    for lq, lk, d in [(1, 1, 1), (3, 5, 4), (8, 8, 16), (5, 17, 9)]:
        q, k, v = rnd(lq, d), rnd(lk, d), rnd(lk, d)
        assert np.max(np.abs(attn_loop(q, k, v) - attn_fp64(q, k, v))) <= 1e-12


def test_matches_torch_cpu_sdpa():
    q, k, v = rnd(2, 3, 37, 24), rnd(2, 3, 29, 24), rnd(2, 3, 29, 24)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    ).numpy()
    assert np.max(np.abs(attn_fp64(q, k, v) - ref)) <= 1e-12


def test_custom_scale():
    q, k, v = rnd(4, 8), rnd(6, 8), rnd(6, 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=0.3
    )[0].numpy()
    assert np.max(np.abs(attn_fp64(q, k, v, scale=0.3) - ref)) <= 1e-12


# ---------------------------------------------------------------- gathers

B, H, F, S, D, L = 2, 3, 4, 6, 8, 5


def video():
    return rnd(B, H, F, S, D), rnd(B, H, F, S, D), rnd(B, H, F, S, D)


def test_spatial_per_sequence_loops():
    q, k, v = video()
    o = spatial(q, k, v)
    for b in range(B):
        for h in range(H):
            for f in range(F):
                ref = attn_loop(q[b, h, f], k[b, h, f], v[b, h, f])
                assert np.max(np.abs(o[b, h, f] - ref)) <= 1e-12


def test_temporal_per_sequence_loops():
    q, k, v = video()
    o = temporal(q, k, v)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                ref = attn_loop(q[b, h, :, s], k[b, h, :, s], v[b, h, :, s])
                assert np.max(np.abs(o[b, h, :, s] - ref)) <= 1e-12


def test_cross_per_head_loops():
    q = rnd(B, H, F, S, D)
    kt, vt = rnd(B, H, L, D), rnd(B, H, L, D)
    o = cross(q, kt, vt)
    assert o.shape == q.shape
    for b in range(B):
        for h in range(H):
            ref = attn_loop(q[b, h].reshape(-1, D), kt[b, h], vt[b, h])
            assert np.max(np.abs(o[b, h].reshape(-1, D) - ref)) <= 1e-12


def test_spatial_locality():
    q, k, v = video()
    o = spatial(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 1:] += 5.0
    v2[:, :, 1:] -= 3.0
    o2 = spatial(q, k2, v2)
    assert np.array_equal(o[:, :, 0], o2[:, :, 0])      # frame 0 untouched
    assert not np.allclose(o[:, :, 1:], o2[:, :, 1:])


def test_temporal_locality():
    q, k, v = video()
    o = temporal(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :, 1:] += 5.0
    v2[:, :, :, 1:] -= 3.0
    o2 = temporal(q, k2, v2)
    assert np.array_equal(o[:, :, :, 0], o2[:, :, :, 0])  # position 0 untouched
    assert not np.allclose(o[:, :, :, 1:], o2[:, :, :, 1:])


def test_single_key_gathers():
    q, k, v = rnd(1, 2, 1, 5, 8), rnd(1, 2, 1, 5, 8), rnd(1, 2, 1, 5, 8)
    assert np.array_equal(temporal(q, k, v), v)            # F = 1
    q, k, v = rnd(1, 2, 5, 1, 8), rnd(1, 2, 5, 1, 8), rnd(1, 2, 5, 1, 8)
    assert np.array_equal(spatial(q, k, v), v)             # S = 1
    q = rnd(1, 2, 3, 4, 8)
    kt, vt = rnd(1, 2, 1, 8), rnd(1, 2, 1, 8)
    o = cross(q, kt, vt)                                   # L = 1
    assert np.array_equal(o, np.broadcast_to(vt[:, :, :, None, :], o.shape))


def test_sampled_forms_match_full():
    q, k, v = video()
    o = spatial(q, k, v)
    assert np.max(np.abs(spatial_rows(q, k, v, 1, 2, 3, [0, 4, 5]) - o[1, 2, 3, [0, 4, 5]])) <= 1e-13
    o = temporal(q, k, v)
    got = temporal_positions(q, k, v, 0, 1, [2, 5])
    assert np.max(np.abs(got - o[0, 1][:, [2, 5]])) <= 1e-13
    kt, vt = rnd(B, H, L, D), rnd(B, H, L, D)
    o = cross(q, kt, vt).reshape(B, H, F * S, D)
    got = cross_rows(q.reshape(B, H, F * S, D), kt, vt, 1, 0, [0, 7, 23])
    assert np.max(np.abs(got - o[1, 0, [0, 7, 23]])) <= 1e-13


def test_bf16_inputs_widen_exactly():
    x = torch.randn(3, 8).to(torch.bfloat16)
    k = torch.randn(4, 8).to(torch.bfloat16)
    v = torch.randn(4, 8).to(torch.bfloat16)
    o1 = attn_fp64(x, k, v)
    o2 = attn_fp64(x.double().numpy(), k.double().numpy(), v.double().numpy())
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------- text padding

def test_cross_text_padding_ignores_pad_tokens():
    # Padding tokens past an entry's text length take no part: whatever they
    # hold (here huge values that would dominate any softmax) the output is
    # the same as with the padding zeroed.
    q = rnd(2, 2, F, S, D)
    kt, vt = rnd(2, 2, L, D), rnd(2, 2, L, D)
    lens = [L - 2, 1]
    o = cross(q, kt, vt, text_len=lens)
    k2, v2 = kt.copy(), vt.copy()
    for b, n in enumerate(lens):
        k2[b, :, n:] = 1e6
        v2[b, :, n:] = -1e6
    assert np.array_equal(cross(q, k2, v2, text_len=lens), o)
    # One real token: every query returns that token's value row exactly.
    for h in range(2):
        assert np.array_equal(o[1, h], np.broadcast_to(vt[1, h, 0], o[1, h].shape))
    # Full length is the unmasked call.
    assert np.max(np.abs(cross(q, kt, vt, text_len=[L, L]) - cross(q, kt, vt))) == 0.0


def test_cross_text_padding_matches_torch_masked_sdpa():
    # Library pin: torch CPU fp64 SDPA with a boolean key mask.
    q = rnd(2, 3, 1, 11, 16)
    kt, vt = rnd(2, 3, 9, 16), rnd(2, 3, 9, 16)
    lens = [4, 9]
    mask = torch.zeros(2, 1, 1, 9, dtype=torch.bool)
    for b, n in enumerate(lens):
        mask[b, :, :, :n] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.reshape(2, 3, 11, 16)), torch.from_numpy(kt), torch.from_numpy(vt),
        attn_mask=mask).numpy()
    got = cross(q, kt, vt, text_len=lens).reshape(2, 3, 11, 16)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_cross_text_padding_rejects_bad_lengths():
    q = rnd(1, 1, 1, 3, 8)
    kt, vt = rnd(1, 1, 5, 8), rnd(1, 1, 5, 8)
    for bad in ([0], [6], [1, 1]):
        with pytest.raises(ValueError):
            cross(q, kt, vt, text_len=bad)
