"""GPU parity on seeded random shapes, through the C ABI, against the fp64
oracle: every kernel family over shapes drawn across its whole supported
range (head widths 8..128, one to many tiles, ragged tails, one token, one
frame, one text token, padded prompts), beyond the hand-picked cases of the
other files.  The draws are fixed by the seed, so a failure names a
reproducible case.

Tolerances as in the other parity tests: attention outputs bf16 max-abs <=
2e-2 and rel-L2 <= 5e-3, fp32 <= 1e-5; projections (a single bf16 rounding
of an fp32-accumulated product) max-abs <= 2^-8 max|ref| and rel-L2 <= 2^-8.
"""

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import lib, synth

pytestmark = pytest.mark.gpu

N_CASES = 48
HEAD_DIMS = list(range(8, 129, 8))


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    return torch.device("cuda:0")


def _check(got, ref, dtype, label):
    got = got.detach().cpu().double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    mx = float(np.abs(err).max())
    rl = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    print(f"[parity] {label} max_abs={mx:.3e} rel_l2={rl:.3e}", flush=True)
    if dtype == "bf16":
        assert mx <= 2e-2 and rl <= 5e-3, (label, mx, rl)
    else:
        assert mx <= 1e-5 and rl <= 1e-5, (label, mx, rl)


def _draw(kind, i):
    """Shape i of a kernel family (deterministic)."""
    rng = np.random.default_rng(1000 * {"spatial": 1, "temporal": 2, "cross": 3, "masked": 4,
                                        "proj": 5}[kind] + i)
    D = int(rng.choice(HEAD_DIMS))
    dt = "f32" if i % 6 == 5 else "bf16"
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    if kind == "spatial":
        F = int(rng.integers(1, 4))
        S = int(rng.choice([1, 2, 31, 32, 33])) if i < 3 else int(rng.integers(1, 700))
        while B * H * F * S * S * D > 1.5e9:
            S //= 2
        return (B, H, F, max(S, 1), D, dt)
    if kind == "temporal":
        F = int(rng.integers(1, 65))
        S = int(rng.integers(1, 300))
        return (B, H, F, S, D, dt)
    F, S = int(rng.integers(1, 4)), int(rng.integers(1, 500))
    L = int(rng.choice([1, 2, 16, 33, 64, 77, 120, 128])) if i < 8 else int(rng.integers(1, 129))
    if kind == "cross":
        return (B, H, F, S, L, D, dt)
    if kind == "masked":
        B = int(rng.integers(2, 4))
        lens = tuple(int(x) for x in rng.integers(1, L + 1, size=B))
        return (B, H, F, S, L, D, lens, dt)
    # proj: hidden size a multiple of 32
    while (H * D) % 32:
        D = int(rng.choice(HEAD_DIMS))
    n_out = int(rng.integers(1, 4))
    return (B, F, S, H, D, n_out)


def _qkv(shape, kv_shape, dt, seed, t):
    q = synth.cpu_tensor(shape, seed, 0, t, 0, 3, 10, dt)
    k = synth.cpu_tensor(kv_shape, seed, 0, t, 1, 3, 10, dt)
    v = synth.cpu_tensor(kv_shape, seed, 0, t, 2, 3, 10, dt)
    return q, k, v


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_spatial(i):
    _dev()
    B, H, F, S, D, dt = case = _draw("spatial", i)
    print(f"[case] spatial {case}", flush=True)
    q, k, v = _qkv((B, H, F, S, D), (B, H, F, S, D), dt, 100 + i, 0)
    ref = oracle.spatial(q, k, v)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qd)
    lib.pab_attn_spatial(qd, kd, vd, o)
    torch.cuda.synchronize()
    _check(o, ref, dt, f"spatial {case}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_temporal(i):
    _dev()
    B, H, F, S, D, dt = case = _draw("temporal", i)
    print(f"[case] temporal {case}", flush=True)
    q, k, v = _qkv((B, H, F, S, D), (B, H, F, S, D), dt, 200 + i, 1)
    ref = oracle.temporal(q, k, v)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qd)
    lib.pab_attn_temporal(qd, kd, vd, o)
    torch.cuda.synchronize()
    _check(o, ref, dt, f"temporal {case}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_cross(i):
    _dev()
    B, H, F, S, L, D, dt = case = _draw("cross", i)
    print(f"[case] cross {case}", flush=True)
    q, k, v = _qkv((B, H, F, S, D), (B, H, L, D), dt, 300 + i, 2)
    ref = oracle.cross(q, k, v)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qd)
    lib.pab_attn_cross(qd, kd, vd, o)
    torch.cuda.synchronize()
    _check(o, ref, dt, f"cross {case}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_masked_cross(i):
    _dev()
    B, H, F, S, L, D, lens, dt = case = _draw("masked", i)
    print(f"[case] masked cross {case}", flush=True)
    q, k, v = _qkv((B, H, F, S, D), (B, H, L, D), dt, 400 + i, 2)
    ref = oracle.cross(q, k, v, text_len=lens)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    for b, n in enumerate(lens):  # padding rows must never be read
        kd[b, :, n:] = float("nan")
        vd[b, :, n:] = float("nan")
    o = torch.empty_like(qd)
    lib.pab_attn_cross_masked(qd, kd, vd, o, lens)
    torch.cuda.synchronize()
    _check(o, ref, dt, f"masked cross {case}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_projections(i):
    _dev()
    B, F, S, H, D, n = case = _draw("proj", i)
    print(f"[case] projections {case}", flush=True)
    C_ = H * D
    g = torch.Generator().manual_seed(500 + i)
    x = torch.randn((B, F * S, C_), generator=g).to(torch.bfloat16)
    w = (torch.randn((n * C_, C_), generator=g) * C_ ** -0.5).to(torch.bfloat16)
    wo = (torch.randn((C_, C_), generator=g) * C_ ** -0.5).to(torch.bfloat16)
    ref_in = oracle.proj_in(x, w, H, D, F, S)
    outs = [torch.empty((B, H, F, S, D), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    lib.pab_proj_in(x.cuda(), w.cuda(), outs, F, S, H, D)
    o = synth.cpu_tensor((B, H, F, S, D), 600 + i, 0, 0, 0, 3, 10, "bf16")
    ref_out = oracle.proj_out(o, wo)
    y = torch.empty((B, F * S, C_), dtype=torch.bfloat16, device="cuda")
    lib.pab_proj_out(o.cuda(), wo.cuda(), y)
    torch.cuda.synchronize()
    tol = 2.0 ** -8
    for got, ref, lab in [(outs[j], ref_in[j], f"proj_in[{j}]") for j in range(n)] + \
            [(y, ref_out, "proj_out")]:
        g_ = got.detach().cpu().double().numpy()
        err = g_ - ref
        mx = float(np.abs(err).max()) / float(np.abs(ref).max())
        rl = float(np.linalg.norm(err) / np.linalg.norm(ref))
        print(f"[parity] {lab} {case} max_abs/max|ref|={mx:.2e} rel_l2={rl:.2e}", flush=True)
        assert mx <= tol and rl <= tol, (lab, case, mx, rl)
