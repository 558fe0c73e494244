"""GPU parity of the projections around an attention (pab_proj_in,
pab_proj_out) against the fp64 oracle, through the C ABI.

PAB article, "Implementation": a broadcast step reuses the attention
module's output, so the module's input and output projections are skipped
with the attention; on a recompute step they run around it.

Tolerance, from the arithmetic: inputs are exact bf16, products accumulate
in fp32 over K <= 1152 terms (relative error far below 2^-16 here), and the
result is rounded once to bf16 (relative error <= 2^-9).  The test bound is
twice that: every element within 2^-8 * max|ref| and the relative L2 error
within 2^-8.
"""

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import lib

pytestmark = pytest.mark.gpu
TOL = 2.0 ** -8


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    return torch.device("cuda:0")


def _check(got, ref, label):
    got = got.detach().float().cpu().double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    mx = float(np.abs(err).max()) / float(np.abs(ref).max())
    rl = float(np.linalg.norm(err) / np.linalg.norm(ref))
    print(f"[parity] {label}: max_abs/max|ref|={mx:.2e} rel_l2={rl:.2e}", flush=True)
    assert mx <= TOL and rl <= TOL, (label, mx, rl)


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


PROJ_IN_CASES = [
    # B, F, S, H, D, n_out
    (1, 2, 100, 4, 64, 3),     # 200 tokens: one ragged token tile
    (2, 3, 90, 4, 72, 3),      # C = 288: the last feature tile is ragged
    (1, 1, 300, 2, 128, 2),    # k, v of a text-like input
    (2, 1, 257, 3, 32, 1),     # q only
]


@pytest.mark.parametrize("case", PROJ_IN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_proj_in_parity(case):
    dev = _dev()
    B, F, S, H, D, n = case
    C = H * D
    print(f"[case] proj_in {case}", flush=True)
    x = _rand((B, F * S, C), 1)
    w = _rand((n * C, C), 2, C ** -0.5)
    refs = oracle.proj_in(x, w, H, D, F, S)
    outs = [torch.full((B, H, F, S, D), float("nan"), dtype=torch.bfloat16, device=dev)
            for _ in range(n)]
    lib.pab_proj_in(x.to(dev), w.to(dev), outs, F, S, H, D)
    torch.cuda.synchronize()
    for i in range(n):
        _check(outs[i], refs[i], f"proj_in {case} out{i}")


PROJ_OUT_CASES = [
    # B, F, S, H, D
    (1, 2, 100, 4, 64),
    (2, 3, 90, 4, 72),
    (1, 1, 300, 2, 128),
]


@pytest.mark.parametrize("case", PROJ_OUT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_proj_out_parity(case):
    dev = _dev()
    B, F, S, H, D = case
    C = H * D
    print(f"[case] proj_out {case}", flush=True)
    o = _rand((B, H, F, S, D), 3)
    w = _rand((C, C), 4, C ** -0.5)
    ref = oracle.proj_out(o, w)
    y = torch.full((B, F * S, C), float("nan"), dtype=torch.bfloat16, device=dev)
    lib.pab_proj_out(o.to(dev), w.to(dev), y)
    torch.cuda.synchronize()
    _check(y, ref, f"proj_out {case}")


def test_proj_full_size_sampled():
    # 480p-latent block: 76 320 tokens, C = 16 x 72 = 1152; q/k/v projection
    # and output projection, checked on sampled tokens.
    dev = _dev()
    B, F, S, H, D = 1, 48, 1590, 16, 72
    C, T = H * D, 48 * 1590
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn((B, T, C), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((3 * C, C), generator=g, device=dev) * C ** -0.5).to(torch.bfloat16)
    q, k, v = (torch.empty((B, H, F, S, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    lib.pab_proj_in(x, w, [q, k, v], F, S, H, D)
    wo = (torch.randn((C, C), generator=g, device=dev) * C ** -0.5).to(torch.bfloat16)
    y = torch.empty((B, T, C), dtype=torch.bfloat16, device=dev)
    lib.pab_proj_out(q, wo, y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, T, 997), [T - 1]]))
    xr = x[0, rows].cpu()
    ref = oracle.linear(xr, w.cpu())                       # [rows, 3C]
    got = torch.stack([t[0].permute(1, 2, 0, 3).reshape(T, C)[rows] for t in (q, k, v)], 1)
    _check(got.reshape(len(rows), 3 * C), ref, "proj_in 480p sampled")
    qr = q[0].permute(1, 2, 0, 3).reshape(T, C)[rows].cpu()
    _check(y[0, rows], oracle.linear(qr, wo.cpu()), "proj_out 480p sampled")
