"""GPU tests of the device workload generator (include/pab_synth.h) against
its host restatement in ``synth``: the Philox4x32-10 words bit for bit, the
Box-Muller normals to fp32 rounding, the perturbed and rounded tensors the
workloads use, and a ragged tail.  Philox4x32-10: Salmon et al., SC'11."""

import numpy as np
import pytest
import torch

from reuse_pab_plan_amd import lib, synth

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    return torch.device("cuda:0")


def _words(t):
    return t.cpu().numpy().view(np.uint32).reshape(-1, 4)


@pytest.mark.parametrize("key,block0,nblocks", [
    (0, 0, 1), (1, 0, 4096), (synth.stream_id(4, 27, 2, 2, 29), 0, 100_003),
    (0xFFFFFFFFFFFFFFFF, 2**32 - 5, 10), (0x0123456789ABCDEF, 2**40 + 1, 777),
])
def test_philox_words_bit_exact(key, block0, nblocks):
    dev = _dev()
    print(f"[case] philox key={key:#x} block0={block0} n={nblocks}", flush=True)
    out = torch.empty(4 * nblocks, dtype=torch.int32, device=dev)
    lib.pab_synth_philox(out, key, block0)
    torch.cuda.synchronize()
    assert np.array_equal(_words(out), synth.philox_blocks(key, block0, nblocks))


def test_normals_match_host_definition():
    # fp32 device log2/sqrt/sin/cos against a float64 evaluation of the same
    # words: agreement to a few fp32 ulps of the result's scale (|z| <= 5.8).
    dev = _dev()
    n = 1 << 20
    key = synth.stream_id(2, 0, 1, 0, -1)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    lib.pab_synth_normal(out, key, 1.0)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    want = synth.philox_normals(key, n)
    err = np.abs(got - want)
    print(f"[parity] normals max abs err {err.max():.2e}", flush=True)
    assert err.max() <= 1e-5
    assert abs(got.mean()) < 5 / np.sqrt(n) and abs(got.var() - 1) < 5 * np.sqrt(2 / n)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 65536 * 3 + 5])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_perturbed_tensor(n, dt):
    # out = round(N_base + sigma N_step): fp32 agreement, and at most one
    # bf16 rounding step apart where the fp32 sums straddle a rounding edge.
    dev = _dev()
    kb, ke, sig = synth.stream_id(3, 1, 2, 1, -1), synth.stream_id(3, 1, 2, 1, 4), 0.02
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.empty(n, dtype=tdt, device=dev)
    lib.pab_synth_normal(out, kb, 1.0, ke, sig)
    torch.cuda.synchronize()
    want = synth.philox_normals(kb, n) + sig * synth.philox_normals(ke, n)
    got = out.cpu().double().numpy()
    if dt == "f32":
        assert np.abs(got - want).max() <= 2e-5
    else:
        # The device's fp32 sum is within eps = 2e-5 of the exact one (the
        # fp32 case above); rounding each to bf16 moves it by at most half a
        # bf16 step (2^-8 relative), so the two roundings differ by at most
        # eps plus one step of the larger magnitude.
        ref = torch.from_numpy(want).float().to(torch.bfloat16).double().numpy()
        eps = 2e-5
        assert (np.abs(got - ref) <= (np.abs(want) + eps) * 2.0 ** -7 + eps).all()
        assert np.mean(got == ref) > 0.99


def test_gpu_tensor_recipe():
    # synth.gpu_tensor: the base alone without perturbation, base + sigma eps
    # with it; the same bytes when drawn twice.
    dev = _dev()
    shape = (1, 2, 3, 37, 72)
    a = synth.gpu_tensor(shape, 2, 0, 0, 1, 10, 30, "bf16", dev)
    b = synth.gpu_tensor(shape, 2, 0, 0, 1, 10, 30, "bf16", dev)
    base = synth.gpu_tensor(shape, 2, 0, 0, 1, 10, 30, "bf16", dev, perturb=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    d = (a.double() - base.double()).cpu().numpy()
    # inner step: sigma = 0.02, so the perturbation is small but present
    assert 0.005 < d.std() < 0.05
    n = int(np.prod(shape))
    want = synth.philox_normals(synth.stream_id(2, 0, 0, 1, -1), n)
    got = base.cpu().double().numpy().reshape(-1)
    assert np.abs(got - want).max() <= np.abs(want).max() * 2.0 ** -8
