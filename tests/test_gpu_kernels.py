"""GPU parity of each libpab.so kernel against the fp64 oracle, through the C
ABI, at sizes the oracle finishes in seconds that still span several tiles
and ragged tails, plus the degenerate cases (a single key returns V
bitwise), dtype coverage and bitwise determinism.

Tolerances (from the stated acceptance bar): bf16 outputs max-abs <= 2e-2 and
rel-L2 <= 5e-3 over the whole output tensor; fp32 outputs <= 1e-5 on both;
MSE relative error <= 1e-6 (exactly 0 when the oracle gives 0).
"""

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import lib, synth

pytestmark = pytest.mark.gpu

BF16_MAXABS, BF16_RELL2 = 2e-2, 5e-3
F32_TOL = 1e-5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    return torch.device("cuda:0")


def metrics(got, ref):
    got = got.detach().cpu().double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    return float(np.abs(err).max()), float(np.linalg.norm(err) / np.linalg.norm(ref))


def assert_close(got, ref, dtype, label=""):
    mx, rl = metrics(got, ref)
    print(f"[parity] {label} max_abs={mx:.3e} rel_l2={rl:.3e}", flush=True)
    if dtype == "bf16":
        assert mx <= BF16_MAXABS and rl <= BF16_RELL2, (label, mx, rl)
    else:
        assert mx <= F32_TOL and rl <= F32_TOL, (label, mx, rl)


def inputs(shape, dtype, seed, type_idx, step=3, n_steps=10, kv_shape=None):
    kv_shape = kv_shape or shape
    q = synth.cpu_tensor(shape, seed, 0, type_idx, 0, step, n_steps, dtype)
    k = synth.cpu_tensor(kv_shape, seed, 0, type_idx, 1, step, n_steps, dtype)
    v = synth.cpu_tensor(kv_shape, seed, 0, type_idx, 2, step, n_steps, dtype)
    return q, k, v


def to_dev(*ts):
    return [t.to("cuda:0").contiguous() for t in ts]


SPATIAL_CASES = [
    # B, H, F, S, D, dtype
    (1, 2, 3, 300, 72, "bf16"),     # last block of 44 rows (one 32-row block per wave), ragged key tiles
    (2, 1, 2, 128, 64, "bf16"),     # exact tiles
    (1, 1, 2, 77, 128, "bf16"),     # widest head
    (1, 3, 1, 200, 8, "bf16"),      # narrowest head (D % 16 == 8)
    (1, 1, 2, 456, 72, "bf16"),     # last block of 200 rows: two 32-row blocks per wave, one idle wave
    (1, 1, 1, 1000, 120, "bf16"),
    (1, 2, 2, 33, 16, "bf16"),
    (1, 4, 4, 64, 64, "f32"),       # tiny-config shape
    (1, 2, 2, 130, 72, "f32"),
    (1, 2, 3, 1, 72, "bf16"),       # one token: the output is V
    (1, 1, 1, 2, 64, "bf16"),
    (1, 1, 2, 1, 64, "f32"),
]


@pytest.mark.parametrize("case", SPATIAL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_spatial_parity(case):
    _dev()
    B, H, F, S, D, dt = case
    print(f"[case] spatial {case}", flush=True)
    q, k, v = inputs((B, H, F, S, D), dt, 21, 0)
    ref = oracle.spatial(q, k, v)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lib.pab_attn_spatial(qd, kd, vd, o)
    torch.cuda.synchronize()
    assert_close(o, ref, dt, f"spatial {case}")


TEMPORAL_CASES = [
    (1, 2, 48, 37, 72, "bf16"),     # 480p frame count, ragged positions
    (1, 2, 32, 20, 72, "bf16"),     # 720p frame count
    (2, 1, 64, 9, 64, "bf16"),      # maximum F
    (1, 1, 33, 12, 128, "bf16"),    # F just above one 32-frame block
    (1, 3, 4, 64, 64, "bf16"),
    (1, 1, 17, 5, 8, "bf16"),
    (1, 4, 4, 64, 64, "f32"),       # tiny-config shape
    (1, 2, 48, 9, 72, "f32"),
    (1, 2, 1, 40, 72, "bf16"),      # one frame: the output is V
    (1, 1, 2, 1, 64, "bf16"),       # one token position
    (1, 1, 1, 3, 64, "f32"),
]


@pytest.mark.parametrize("case", TEMPORAL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_temporal_parity(case):
    _dev()
    B, H, F, S, D, dt = case
    print(f"[case] temporal {case}", flush=True)
    q, k, v = inputs((B, H, F, S, D), dt, 22, 1)
    ref = oracle.temporal(q, k, v)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lib.pab_attn_temporal(qd, kd, vd, o)
    torch.cuda.synchronize()
    assert_close(o, ref, dt, f"temporal {case}")


CROSS_CASES = [
    # B, H, F, S, L, D, dtype
    (1, 2, 3, 100, 120, 72, "bf16"),   # ragged query tiles, 120 text tokens
    (2, 2, 1, 513, 120, 64, "bf16"),
    (1, 1, 2, 64, 128, 128, "bf16"),   # maximum L
    (1, 2, 1, 50, 16, 72, "bf16"),
    (1, 1, 1, 40, 33, 8, "bf16"),
    (1, 4, 4, 64, 16, 64, "f32"),      # tiny-config shape
    (1, 2, 2, 70, 120, 72, "f32"),
    (1, 1, 2, 45, 1, 72, "bf16"),      # one text token: the output is its V row
    (1, 2, 1, 1, 1, 64, "bf16"),       # one query, one text token
    (1, 1, 1, 3, 1, 64, "f32"),
    # No bias column (D % 16 == 0) and 65..96 text tokens: four 32-key blocks,
    # of which the third holds the last real keys and the fourth none.  Keys
    # from L on must be masked in both (a ones row, D % 32 == 0, would
    # otherwise count them in the denominator).
    (2, 3, 2, 415, 69, 96, "bf16"),
    (1, 2, 1, 100, 96, 64, "bf16"),
    (1, 1, 1, 64, 65, 32, "bf16"),
    (1, 1, 2, 50, 80, 128, "bf16"),
    (1, 2, 1, 40, 70, 48, "bf16"),
]


@pytest.mark.parametrize("case", CROSS_CASES, ids=lambda c: "x".join(map(str, c)))
def test_cross_parity(case):
    _dev()
    B, H, F, S, L, D, dt = case
    print(f"[case] cross {case}", flush=True)
    q, k, v = inputs((B, H, F, S, D), dt, 23, 2, kv_shape=(B, H, L, D))
    ref = oracle.cross(q, k, v)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lib.pab_attn_cross(qd, kd, vd, o)
    torch.cuda.synchronize()
    assert_close(o, ref, dt, f"cross {case}")


MASKED_CROSS_CASES = [
    # B, H, F, S, L, D, text_len, dtype
    (2, 2, 2, 100, 120, 72, (77, 1), "bf16"),    # CFG: padded prompt + empty prompt
    (2, 2, 1, 130, 120, 64, (50, 120), "bf16"),  # no bias column: score masking path
    (2, 1, 1, 90, 120, 72, (120, 120), "bf16"),  # nothing padded: the single-launch path
    (3, 1, 1, 70, 33, 8, (33, 2, 17), "bf16"),
    (2, 4, 4, 64, 16, 64, (16, 5), "f32"),       # tiny-config shape
    (2, 2, 1, 90, 120, 64, (70, 96), "bf16"),    # no bias column, 65..96 real tokens
    (2, 1, 1, 60, 100, 96, (65, 100), "bf16"),
]


@pytest.mark.parametrize("case", MASKED_CROSS_CASES, ids=lambda c: "x".join(map(str, c[:6])) + "-" + c[7])
def test_masked_cross_parity(case):
    # Padded prompts (pab_attn_cross_masked): entry b attends to its first
    # text_len[b] tokens.  The padding rows are filled with huge values and
    # NaN on the device: they must not be read.
    _dev()
    B, H, F, S, L, D, lens, dt = case
    print(f"[case] masked cross {case}", flush=True)
    q, k, v = inputs((B, H, F, S, D), dt, 29, 2, kv_shape=(B, H, L, D))
    ref = oracle.cross(q, k, v, text_len=lens)
    qd, kd, vd = to_dev(q, k, v)
    for b, n in enumerate(lens):
        kd[b, :, n:] = float("nan")
        vd[b, :, n:] = 1e30
    o = torch.empty_like(qd)
    lib.pab_attn_cross_masked(qd, kd, vd, o, lens)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert_close(o, ref, dt, f"masked cross {case}")
    for b, n in enumerate(lens):
        if n == 1:  # a single real text token returns its value row exactly
            assert torch.equal(o[b], vd[b, :, :1, None, :].expand_as(o[b]))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_key_returns_v_bitwise(dt):
    _dev()
    # spatial with S = 1, temporal with F = 1, cross with L = 1
    q, k, v = to_dev(*inputs((1, 2, 3, 1, 72), dt, 5, 0))
    o = torch.empty_like(q)
    lib.pab_attn_spatial(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    q, k, v = to_dev(*inputs((1, 2, 1, 45, 64), dt, 6, 1))
    o = torch.empty_like(q)
    lib.pab_attn_temporal(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    q, k, v = to_dev(*inputs((1, 2, 2, 50, 72), dt, 7, 2, kv_shape=(1, 2, 1, 72)))
    o = torch.empty_like(q)
    lib.pab_attn_cross(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.equal(o, v[:, :, :, None, :].expand_as(o))


def test_custom_scale():
    _dev()
    q, k, v = inputs((1, 2, 2, 150, 72), "bf16", 8, 0)
    ref = oracle.spatial(q, k, v, scale=0.05)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lib.pab_attn_spatial(qd, kd, vd, o, softmax_scale=0.05)
    torch.cuda.synchronize()
    assert_close(o, ref, "bf16", "spatial scale=0.05")


LARGE_LOGIT_CASES = [
    # kind, B x H x F x S x D, text tokens, multiplier on Q
    ("spatial", (1, 1, 1, 700, 64), None, 6.0),    # later keys above the first unit's max
    ("spatial", (1, 2, 2, 333, 72), None, 30.0),
    ("temporal", (1, 2, 48, 37, 72), None, 30.0),  # full-row max over the frames
    ("cross", (1, 2, 2, 150, 64), 100, 30.0),      # no bias column, padded key blocks
    ("cross", (1, 1, 3, 90, 72), 120, 30.0),       # bias column
]


@pytest.mark.parametrize("case", LARGE_LOGIT_CASES, ids=lambda c: f"{c[0]}-{'x'.join(map(str, c[1]))}")
def test_large_logits_stable(case):
    # Scores spanning hundreds to thousands of units in the log domain.
    _dev()
    kind, shape, L, mult = case
    print(f"[case] large logits {case}", flush=True)
    kv = (shape[0], shape[1], L, shape[4]) if kind == "cross" else None
    q, k, v = inputs(shape, "bf16", 9, 0, kv_shape=kv)
    q = (q.float() * mult).to(torch.bfloat16)
    ref = getattr(oracle, kind)(q, k, v)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    getattr(lib, f"pab_attn_{kind}")(qd, kd, vd, o)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert_close(o, ref, "bf16", f"{kind} large logits")


def test_determinism_bitwise():
    _dev()
    q, k, v = to_dev(*inputs((1, 2, 4, 333, 72), "bf16", 10, 0))
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    for fn in (lib.pab_attn_spatial, lib.pab_attn_temporal):
        fn(q, k, v, o1)
        fn(q, k, v, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    kt, vt = k[:, :, 0, :120].contiguous(), v[:, :, 0, :120].contiguous()
    lib.pab_attn_cross(q, kt, vt, o1)
    lib.pab_attn_cross(q, kt, vt, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_guard_bands_untouched():
    # Output written into the middle of a larger NaN-filled buffer: nothing
    # outside the output region may change.
    _dev()
    B, H, F, S, D = 1, 2, 3, 130, 72
    q, k, v = to_dev(*inputs((B, H, F, S, D), "bf16", 11, 0))
    n = q.numel()
    pad = 4096
    for fn in (lib.pab_attn_spatial, lib.pab_attn_temporal):
        buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        o = buf[pad:pad + n].view(B, H, F, S, D)
        fn(q, k, v, o)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n:].float()).all()
        assert torch.isfinite(o.float()).all()
    kt, vt = k[:, :, 0, :100].contiguous(), v[:, :, 0, :100].contiguous()
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    o = buf[pad:pad + n].view(B, H, F, S, D)
    lib.pab_attn_cross(q, kt, vt, o)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n:].float()).all()
    assert torch.isfinite(o.float()).all()


# ------------------------------------------------------------------- MSE

@pytest.mark.parametrize("n", [1, 7, 1000, 65536, 65536 * 3 + 5, 2_000_003])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_mse_parity(n, dt):
    _dev()
    print(f"[case] mse n={n} {dt}", flush=True)
    a = synth.cpu_tensor((n,), 31, 0, 0, 0, 1, 10, dt)
    b = synth.cpu_tensor((n,), 31, 0, 0, 1, 1, 10, dt)
    ref = oracle.mse(a, b)
    ad, bd = to_dev(a, b)
    out = torch.zeros(1, dtype=torch.float64, device="cuda:0")
    ws = torch.empty(lib.pab_mse_workspace_bytes(n), dtype=torch.uint8, device="cuda:0")
    lib.pab_attn_diff_mse(ad, bd, out, ws)
    torch.cuda.synchronize()
    got = float(out.item())
    assert abs(got - ref) <= 1e-6 * ref, (got, ref)
    # identical inputs give exactly zero; repeated calls are bitwise equal
    lib.pab_attn_diff_mse(ad, ad, out, ws)
    torch.cuda.synchronize()
    assert out.item() == 0.0
    lib.pab_attn_diff_mse(ad, bd, out, ws)
    torch.cuda.synchronize()
    assert float(out.item()) == got


def test_mse_exact_dyadic_shift():
    _dev()
    x = torch.randint(-1000, 1000, (123457,), dtype=torch.int32).to(torch.float32)
    y = x + 0.5
    out = torch.zeros(1, dtype=torch.float64, device="cuda:0")
    ws = torch.empty(lib.pab_mse_workspace_bytes(x.numel()), dtype=torch.uint8, device="cuda:0")
    lib.pab_attn_diff_mse(x.cuda(), y.cuda(), out, ws)
    torch.cuda.synchronize()
    assert out.item() == 0.25


@pytest.mark.parametrize("D", [72, 40, 8])
def test_f32_path_ignores_stale_lds(D):
    # The fp32 kernel's tiles have columns past D that are never loaded.  Run
    # a bf16 spatial call over NaN inputs first, on every CU, so the LDS holds
    # NaN bit patterns, then the fp32 call: its output must stay finite and
    # match the oracle (regression test: those columns once read stale LDS).
    dev = _dev()
    junk = torch.full((1, 8, 64, 1590, 72), float("nan"), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(junk)
    lib.pab_attn_spatial(junk, junk, junk, out)
    case = (1, 2, 2, 130, D, "f32")
    q, k, v = inputs(case[:5], "f32", 31, 0)
    ref = oracle.spatial(q, k, v)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lib.pab_attn_spatial(qd, kd, vd, o)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    assert_close(o, ref, "f32", f"spatial {case} after NaN LDS")


def test_cross_text_length_grid():
    # Text lengths around the 32-key block edges (1, 2 or 4 key blocks, the
    # last one or two partly or wholly padding) for head widths with and
    # without a bias column (D % 16) and a ones column (D % 32), plain and
    # padded prompts (padding rows NaN / huge on the device: never read).
    _dev()
    failures = []
    for D in (16, 32, 48, 64, 96, 128):
        for L in (31, 33, 64, 65, 70, 96, 97):
            B, H, F, S = 2, 1, 1, 70
            q, k, v = inputs((B, H, F, S, D), "bf16", 31, 2, kv_shape=(B, H, L, D))
            for lens in (None, (L, max(1, L - 7))):
                ref = oracle.cross(q, k, v, text_len=lens)
                qd, kd, vd = to_dev(q, k, v)
                o = torch.empty_like(qd)
                if lens is None:
                    lib.pab_attn_cross(qd, kd, vd, o)
                else:
                    for b, n in enumerate(lens):
                        kd[b, :, n:] = float("nan")
                        vd[b, :, n:] = 1e30
                    lib.pab_attn_cross_masked(qd, kd, vd, o, lens)
                torch.cuda.synchronize()
                got = o.detach().cpu().double().numpy()
                err = got - np.asarray(ref, np.float64)
                mx = float(np.abs(err).max())
                rl = float(np.linalg.norm(err) / np.linalg.norm(ref))
                if not (np.isfinite(got).all() and mx <= 2e-2 and rl <= 5e-3):
                    failures.append((D, L, lens, mx, rl))
    print(f"[parity] cross text-length grid: {len(failures)} failures", flush=True)
    assert not failures, failures
