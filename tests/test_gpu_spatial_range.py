"""GPU tests of spatial attention's reference maximum and its exact fallback.

Softmax does not change when a constant is subtracted from a row's scores;
the bf16 spatial kernel subtracts, for each row, the maximum of its first 32
scores plus a fixed headroom, and keeps it for the whole row.  A row whose
later scores exceed that by so much that the exponentials leave fp32 range is
recomputed exactly (two-pass fp32 softmax from HBM) by its whole wave.  These
cases plant such a key -- far past the first 32 -- so the fallback runs, for
every wave or for some of them, with and without the attention difference
taken in the output pass, and compare with the fp64 oracle.
"""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import lib, synth

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    return torch.device("cuda:0")


def _planted(B, H, F, S, D, key, rows, seed, q_shift=3.0, k_value=20.0):
    """bf16 q, k, v with key ``key`` of every frame set to k_value in every
    channel and the query rows in ``rows`` shifted by q_shift: their score
    with that key is about D * q_shift * k_value, far above the rest."""
    shape = (B, H, F, S, D)
    q = synth.cpu_tensor(shape, seed, 0, 0, 0, 3, 10, "f32")
    k = synth.cpu_tensor(shape, seed, 0, 0, 1, 3, 10, "f32")
    v = synth.cpu_tensor(shape, seed, 0, 0, 2, 3, 10, "f32")
    q[:, :, :, rows] += q_shift
    k[:, :, :, key] = k_value
    return (t.to(torch.bfloat16) for t in (q, k, v))


def _check(o, ref, label):
    got = o.detach().cpu().double().numpy()
    err = got - ref
    mx = float(np.abs(err).max())
    rl = float(np.linalg.norm(err) / np.linalg.norm(ref))
    print(f"[parity] {label} max_abs={mx:.3e} rel_l2={rl:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert mx <= 2e-2 and rl <= 5e-3, (label, mx, rl)


@pytest.mark.parametrize("D", [72, 64, 128, 40])
def test_late_dominant_key_every_wave(D):
    # Every query row is dominated by key 450: all waves fall back.
    dev = _dev()
    B, H, F, S = 1, 2, 2, 600
    print(f"[case] spatial planted key, all rows, D={D}", flush=True)
    q, k, v = _planted(B, H, F, S, D, 450, slice(None), 41)
    ref = oracle.spatial(q, k, v)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lib.pab_attn_spatial(qd, kd, vd, o)
    torch.cuda.synchronize()
    _check(o, ref, f"planted key D={D}")


@pytest.mark.parametrize("S", [300, 1590])
def test_late_dominant_key_some_waves(S):
    # Only rows 64..127 (the second wave of the first block) and the last 10
    # rows are shifted toward the planted key: their waves fall back, the
    # others keep the fast path, in the same launch.
    dev = _dev()
    B, H, F, D = 1, 1, 2, 72
    rows = np.r_[64:128, S - 10:S]
    print(f"[case] spatial planted key, some rows, S={S}", flush=True)
    q, k, v = _planted(B, H, F, S, D, S - 40, rows, 42)
    ref = oracle.spatial(q, k, v)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lib.pab_attn_spatial(qd, kd, vd, o)
    torch.cuda.synchronize()
    _check(o, ref, f"planted key some rows S={S}")


def test_fallback_with_attention_difference():
    # Two PAB-off steps through the dispatcher with the difference folded into
    # the output pass: the second step's outputs fall back for some waves; the
    # drift must equal the oracle MSE of the two stored outputs.
    dev = _dev()
    B, H, F, S, D = 1, 2, 3, 333, 72
    steps = [_planted(B, H, F, S, D, 300, np.r_[0:64], 43 + i) for i in range(2)]
    rec = np.ones((2, 1), dtype=np.uint8)
    slots = [torch.empty((B, H, F, S, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    drift = torch.full((2,), -1.0, dtype=torch.float64, device=dev)
    ws = torch.empty(lib.pab_mse_workspace_bytes(B * H * F * S * D), dtype=torch.uint8, device=dev)
    types = (lib.TypeDesc * 1)()
    types[0].kind = lib.PAB_SPATIAL
    types[0].slot[0], types[0].slot[1] = slots[0].data_ptr(), slots[1].data_ptr()
    types[0].B, types[0].H, types[0].F, types[0].S, types[0].D = B, H, F, S, D
    types[0].drift = drift.data_ptr()
    desc = lib.StepDesc(num_steps=2, num_types=1,
                        recompute=rec.ctypes.data_as(C.POINTER(C.c_uint8)),
                        types=C.cast(types, C.POINTER(lib.TypeDesc)), dtype=lib.PAB_BF16,
                        softmax_scale=0.0, workspace=ws.data_ptr(), workspace_bytes=ws.numel(),
                        stream=torch.cuda.current_stream().cuda_stream)
    outs = []
    keep = []
    for i, (q, k, v) in enumerate(steps):
        qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
        keep.append((qd, kd, vd))
        types[0].q, types[0].k, types[0].v = qd.data_ptr(), kd.data_ptr(), vd.data_ptr()
        _, ptrs = lib.pab_step_dispatch(desc, i)
        torch.cuda.synchronize()
        out = [s for s in slots if s.data_ptr() == ptrs[0]][0]
        _check(out, oracle.spatial(q, k, v), f"dispatch step {i}")
        outs.append(out.double().cpu().numpy())
    want = oracle.mse(outs[1], outs[0])
    got = float(drift[1].item())
    print(f"[parity] fallback drift got={got:.6e} want={want:.6e}", flush=True)
    assert abs(got - want) <= 1e-6 * want
