"""GPU test of pab_attn_diff_mse_noalloc, the attention-difference MSE for
callers that cannot allocate: through the C ABI, two calls in a row (the
second on a smaller input) against pab_attn_diff_mse with a workspace (the
same kernels and reduction order: bitwise equal) and against the fp64 oracle
MSE (PAB article, Figure 1 caption) within 1e-6 relative."""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import lib, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dt):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = lib.load()
    dev = torch.device("cuda:0")
    ws = torch.empty(lib.pab_mse_workspace_bytes(3_000_017), dtype=torch.uint8, device=dev)
    for n in (3_000_017, 777):  # the second call reuses the scratch on a smaller input
        print(f"[case] mse noalloc {dt} n={n}", flush=True)
        a = synth.cpu_tensor((n,), 61, 0, 0, 0, 2, 10, dt)
        b = synth.cpu_tensor((n,), 61, 0, 0, 1, 2, 10, dt)
        ad, bd = a.to(dev), b.to(dev)
        got = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
        ref = torch.full((1,), -2.0, dtype=torch.float64, device=dev)
        st = L.pab_attn_diff_mse_noalloc(C.c_void_p(ad.data_ptr()), C.c_void_p(bd.data_ptr()), n,
                                         lib.PAB_BF16 if dt == "bf16" else lib.PAB_F32,
                                         C.c_void_p(got.data_ptr()), None)
        assert st == lib.PAB_OK, lib.pab_last_error()
        lib.pab_attn_diff_mse(ad, bd, ref, ws)
        torch.cuda.synchronize()
        want = oracle.mse(a, b)
        g, r = float(got.item()), float(ref.item())
        print(f"[parity] noalloc {dt} n={n}: {g!r} workspace {r!r} oracle {want!r}", flush=True)
        assert g == r
        assert abs(g - want) <= 1e-6 * want


def test_noalloc_binding_and_zero():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    dev = torch.device("cuda:0")
    x = synth.cpu_tensor((4099,), 62, 0, 0, 0, 2, 10, "bf16").to(dev)
    out = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
    lib.pab_attn_diff_mse_noalloc(x, x, out)
    torch.cuda.synchronize()
    assert out.item() == 0.0
