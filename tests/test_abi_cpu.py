"""CPU-side tests of libpab.so: it loads, exports every declared symbol, the
host planner is bit-exact against the oracle, and argument validation
returns the documented codes before any device call (no kernels run here)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import schedule as oracle_schedule
from reuse_pab_plan_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pab.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lib.LIB_PATH), reason="libpab.so not built")


PEAKS_HEADER = os.path.join(ROOT, "include", "pab_peaks.h")
SYNTH_HEADER = os.path.join(ROOT, "include", "pab_synth.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pab_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = lib.load()
    names = declared_functions()
    assert set(names) == set(lib.EXPORTED)
    peaks = declared_functions(PEAKS_HEADER)
    assert set(peaks) == set(lib.EXPORTED_PEAKS)
    synth_fns = declared_functions(SYNTH_HEADER)
    assert set(synth_fns) == set(lib.EXPORTED_SYNTH)
    for name in names + peaks + synth_fns:
        assert hasattr(L, name), name
    assert "gfx950" in lib.pab_version()


def test_peak_helpers_validate_before_launch():
    L = lib.load()
    sink_bytes = int(L.pab_peak_sink_bytes())
    assert sink_bytes >= 65536 * 4
    work = C.c_double(0.0)
    P = lambda *a: (C.c_void_p * len(a))(*[C.c_void_p(x) for x in a])
    sink = C.c_void_p(0x100000)
    src, dst = P(0x1000, 0x100000000), P(0x200000000)
    # no stream / too many streams
    assert L.pab_peak_stream(src, 0, dst, 0, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(src, 5, dst, 0, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(src, 1, dst, 3, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    # size, grid, variant
    assert L.pab_peak_stream(src, 1, dst, 1, 1000, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(src, 1, dst, 1, 1024, 0, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(src, 1, dst, 1, 1024, 70000, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    for variant in (-1, 6, 7, 14, 15, 16):
        assert L.pab_peak_stream(src, 1, dst, 1, 1024, 1024, variant, sink, sink_bytes, None) == \
            lib.PAB_ERR_INVALID_ARG
    # misaligned and overlapping buffers
    assert L.pab_peak_stream(P(0x1008), 1, dst, 1, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(P(0x1000), 1, P(0x1200), 1, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_stream(P(0x1000, 0x1100), 2, dst, 0, 1024, 1024, 0, sink, sink_bytes, None) == lib.PAB_ERR_INVALID_ARG
    # a read-only pass needs a sink of pab_peak_sink_bytes()
    assert L.pab_peak_stream(src, 1, dst, 0, 1024, 1024, 0, sink, 16, None) == lib.PAB_ERR_CAPACITY
    assert L.pab_peak_mfma_bf16(0, sink, sink_bytes, C.byref(work), None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_peak_exp(1, sink, 64, C.byref(work), None) == lib.PAB_ERR_CAPACITY


@pytest.mark.parametrize("win", [(15, 85), (0, 100), (50, 50), (0, 0), (30, 60), (10, 90)])
def test_planner_bit_exact_vs_oracle(win):
    lo, hi = win
    for n in list(range(1, 61)) + [97, 150, 200]:
        for ranges in ([0], [2, 4, 6], [2, 3, 5], [1, 7], [12, 0, 3, 9]):
            r1, s1, c1 = lib.pab_plan_schedule(n, ranges, lo, hi)
            r2, s2, c2 = oracle_schedule(n, ranges, lo, hi)
            assert np.array_equal(r1, r2), (n, ranges, win)
            assert np.array_equal(s1, s2), (n, ranges, win)
            assert np.array_equal(c1, c2), (n, ranges, win)


def test_planner_config_counts():
    # the three benchmark schedules
    assert list(lib.pab_plan_schedule(10, [2, 3, 5])[2]) == [6, 5, 5]
    assert list(lib.pab_plan_schedule(30, [2, 4, 6])[2]) == [16, 14, 12]
    assert list(lib.pab_plan_schedule(50, [2, 6])[2]) == [27, 20]


def test_planner_errors():
    L = lib.load()
    r = (C.c_int32 * 2)(1, 2)
    rec = (C.c_uint8 * 20)()
    assert L.pab_plan_schedule(0, 2, r, 15, 85, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 0, r, 15, 85, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 33, r, 15, 85, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 2, None, 15, 85, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 2, r, 60, 40, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 2, r, -1, 40, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert "lo <= hi" in lib.pab_last_error()
    neg = (C.c_int32 * 2)(1, -2)
    assert L.pab_plan_schedule(10, 2, neg, 15, 85, rec, None, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_plan_schedule(10, 2, r, 15, 85, rec, None, None) == lib.PAB_OK
    assert lib.pab_last_error() == ""


# Fake, never-dereferenced, 16-byte aligned addresses: validation must reject
# every one of these calls before touching the device.
A, B_, Cc, O = 0x10000, 0x20000000, 0x40000000, 0x60000000


def test_attention_validation_codes():
    L = lib.load()
    sp = L.pab_attn_spatial
    args = dict(B=1, H=2, F=3, S=5, D=64, dt=lib.PAB_BF16, sc=0.0)

    def call(fn, q=A, k=B_, v=Cc, o=O, **kw):
        a = {**args, **kw}
        return fn(q, k, v, o, a["B"], a["H"], a["F"], a["S"], a["D"], a["dt"], a["sc"], None)

    assert call(sp, q=None) == lib.PAB_ERR_INVALID_ARG
    assert call(sp, q=A + 8) == lib.PAB_ERR_INVALID_ARG              # misaligned
    assert call(sp, B=0) == lib.PAB_ERR_INVALID_ARG
    assert call(sp, S=-4) == lib.PAB_ERR_INVALID_ARG
    assert call(sp, D=60) == lib.PAB_ERR_UNSUPPORTED                 # not a multiple of 8
    assert call(sp, D=136) == lib.PAB_ERR_UNSUPPORTED
    assert call(sp, dt=7) == lib.PAB_ERR_UNSUPPORTED
    assert call(sp, sc=-1.0) == lib.PAB_ERR_INVALID_ARG
    assert call(sp, sc=float("nan")) == lib.PAB_ERR_INVALID_ARG
    assert call(sp, o=A) == lib.PAB_ERR_INVALID_ARG                  # o aliases q
    assert "overlap" in lib.pab_last_error()
    assert call(L.pab_attn_temporal, F=65) == lib.PAB_ERR_UNSUPPORTED
    # bf16 kernels use 32-bit byte offsets within a sequence / (b, h) slab.
    assert call(sp, B=1, H=1, F=1, S=1 << 24, D=128) == lib.PAB_ERR_UNSUPPORTED
    assert call(L.pab_attn_temporal, B=1, H=1, F=64, S=1 << 19, D=64) == lib.PAB_ERR_UNSUPPORTED
    assert "4 GiB" in lib.pab_last_error()
    cr = L.pab_attn_cross
    cm = L.pab_attn_cross_masked
    lens = (C.c_int32 * 2)(5, 16)
    assert cm(A, B_, Cc, O, 2, 2, 100, 16, 64, 0, 0.0, None, None) == lib.PAB_ERR_INVALID_ARG
    assert "text_len" in lib.pab_last_error()
    for bad in ((0, 16), (5, 17), (-1, 3)):
        lb = (C.c_int32 * 2)(*bad)
        assert cm(A, B_, Cc, O, 2, 2, 100, 16, 64, 0, 0.0, lb, None) == lib.PAB_ERR_INVALID_ARG
        assert "outside [1, L" in lib.pab_last_error()
    assert cm(A, B_, Cc, O, 2, 2, 100, 129, 64, 0, 0.0, lens, None) == lib.PAB_ERR_UNSUPPORTED
    assert cr(A, B_, Cc, O, 1, 2, 100, 129, 64, 0, 0.0, None) == lib.PAB_ERR_UNSUPPORTED  # L > 128
    assert cr(A, B_, Cc, O, 1, 2, 0, 16, 64, 0, 0.0, None) == lib.PAB_ERR_INVALID_ARG
    assert cr(A, B_, Cc, A, 1, 2, 100, 16, 64, 0, 0.0, None) == lib.PAB_ERR_INVALID_ARG


def test_mse_validation_codes():
    L = lib.load()
    n = 1000
    ws = lib.pab_mse_workspace_bytes(n)
    assert ws >= 8 and ws % 256 == 0
    assert lib.pab_mse_workspace_bytes(0) == 0
    big = lib.pab_mse_workspace_bytes(10**9)
    assert big >= 2048 * 8
    assert L.pab_attn_diff_mse(A, B_, n, 0, O, Cc, ws - 8, None) == lib.PAB_ERR_CAPACITY
    assert L.pab_attn_diff_mse(A, B_, 0, 0, O, Cc, ws, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_attn_diff_mse(A, B_, n, 3, O, Cc, ws, None) == lib.PAB_ERR_UNSUPPORTED
    assert L.pab_attn_diff_mse(A + 4, B_, n, 0, O, Cc, ws, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_attn_diff_mse(A, B_, n, 0, O + 4, Cc, ws, None) == lib.PAB_ERR_INVALID_ARG


def test_noalloc_mse_validation_codes():
    # Checked before any device call (no GPU here).
    L = lib.load()
    ok, out = C.c_void_p(0x10000), C.c_void_p(0x20000)
    f = L.pab_attn_diff_mse_noalloc
    assert f(None, ok, 10, lib.PAB_BF16, out, None) == lib.PAB_ERR_INVALID_ARG
    assert f(ok, None, 10, lib.PAB_BF16, out, None) == lib.PAB_ERR_INVALID_ARG
    assert f(ok, ok, 10, lib.PAB_BF16, None, None) == lib.PAB_ERR_INVALID_ARG
    assert f(C.c_void_p(0x10008), ok, 10, lib.PAB_BF16, out, None) == lib.PAB_ERR_INVALID_ARG
    assert f(ok, ok, 10, lib.PAB_BF16, C.c_void_p(0x20004), None) == lib.PAB_ERR_INVALID_ARG
    assert f(ok, ok, 0, lib.PAB_BF16, out, None) == lib.PAB_ERR_INVALID_ARG
    assert f(ok, ok, 10, 5, out, None) == lib.PAB_ERR_UNSUPPORTED
    assert "noalloc" in lib.pab_last_error()


def test_dispatch_validation_codes():
    rec, _, _ = lib.pab_plan_schedule(4, [1])
    t = lib.TypeDesc(kind=9, q=A, k=B_, v=Cc, B=1, H=1, F=1, S=8, D=64, L=0)
    t.slot[0] = O
    types = (lib.TypeDesc * 1)(t)
    d = lib.StepDesc(num_steps=4, num_types=1,
                     recompute=rec.ctypes.data_as(C.POINTER(C.c_uint8)),
                     types=C.cast(types, C.POINTER(lib.TypeDesc)), dtype=0, softmax_scale=0.0)
    L = lib.load()
    assert L.pab_step_dispatch(C.byref(d), 0, None, None) == lib.PAB_ERR_INVALID_ARG  # bad kind
    types[0].kind = lib.PAB_SPATIAL
    assert L.pab_step_dispatch(C.byref(d), 4, None, None) == lib.PAB_ERR_INVALID_ARG  # step range
    assert L.pab_step_dispatch(C.byref(d), -1, None, None) == lib.PAB_ERR_INVALID_ARG
    types[0].D = 12
    assert L.pab_step_dispatch(C.byref(d), 0, None, None) == lib.PAB_ERR_UNSUPPORTED
    types[0].D = 64
    types[0].slot[1] = O + 64   # overlapping second slot
    assert L.pab_step_dispatch(C.byref(d), 0, None, None) == lib.PAB_ERR_INVALID_ARG
    types[0].slot[1] = 0x70000000
    types[0].drift = 0x78000000   # drift without a workspace
    assert L.pab_step_dispatch(C.byref(d), 0, None, None) == lib.PAB_ERR_INVALID_ARG
    d.workspace, d.workspace_bytes = 0x7c000000, 8
    assert L.pab_step_dispatch(C.byref(d), 0, None, None) == lib.PAB_ERR_CAPACITY
    assert L.pab_step_dispatch(None, 0, None, None) == lib.PAB_ERR_INVALID_ARG


def test_dispatch_reuse_step_needs_no_inputs():
    # A type that reuses its slot launches nothing and reads no input: a
    # trajectory resumed at a broadcast step may leave q, k, v NULL.  Nothing
    # here touches the device (no launch at a reuse step).
    rec, src, _ = lib.pab_plan_schedule(4, [1])      # steps 0, 1, 3 compute; 2 reuses 1
    assert rec[2, 0] == 0 and src[2, 0] == 1
    t = (lib.TypeDesc * 1)()
    t[0].kind = lib.PAB_SPATIAL
    t[0].B, t[0].H, t[0].F, t[0].S, t[0].D = 1, 1, 1, 8, 64
    t[0].slot[0], t[0].slot[1] = 0x100000, 0x200000
    d = lib.StepDesc(num_steps=4, num_types=1,
                     recompute=rec.ctypes.data_as(C.POINTER(C.c_uint8)),
                     types=C.cast(t, C.POINTER(lib.TypeDesc)), dtype=lib.PAB_BF16,
                     softmax_scale=0.0, workspace=None, workspace_bytes=0, stream=None)
    L = lib.load()
    mask = C.c_uint32(7)
    ptrs = (C.c_void_p * 1)()
    assert L.pab_step_dispatch(C.byref(d), 2, C.byref(mask), ptrs) == lib.PAB_OK
    # two recomputes so far (steps 0 and 1): the second wrote slot[1]
    assert mask.value == 0 and ptrs[0] == 0x200000
    # a recompute step still needs its inputs
    assert L.pab_step_dispatch(C.byref(d), 3, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG
    # and a reuse step still needs valid slots
    t[0].slot[0] = 0
    assert L.pab_step_dispatch(C.byref(d), 2, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG
    t[0].slot[0] = 0x100008
    assert L.pab_step_dispatch(C.byref(d), 2, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG
    t[0].slot[0] = 0x100000
    t[0].slot[1] = 0x100000 + 64   # overlaps slot[0]
    assert L.pab_step_dispatch(C.byref(d), 2, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG
    t[0].slot[1] = 0x200000
    t[0].S = 0
    assert L.pab_step_dispatch(C.byref(d), 2, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG


def test_dispatch_module_rejects_missing_weights_and_fp32():
    # A module (x set) needs w_in, w_out and four scratch buffers, and is
    # built for bf16 only; every check runs on the host before any launch.
    sched = np.ones((2, 1), dtype=np.uint8)
    for dtype, missing, code in ((lib.PAB_BF16, "w_out", lib.PAB_ERR_INVALID_ARG),
                                 (lib.PAB_F32, None, lib.PAB_ERR_UNSUPPORTED)):
        t = (lib.TypeDesc * 1)()
        t[0].kind = lib.KINDS["spatial"]
        t[0].slot[0], t[0].slot[1] = 0x100000, 0x200000
        t[0].B, t[0].H, t[0].F, t[0].S, t[0].D = 1, 2, 2, 8, 64
        t[0].x, t[0].w_in, t[0].w_out = 0x300000, 0x400000, 0x500000
        for j in range(4):
            t[0].scratch[j] = 0x600000 + j * 0x100000
        if missing:
            setattr(t[0], missing, None)
        d = lib.StepDesc(num_steps=2, num_types=1,
                         recompute=sched.ctypes.data_as(C.POINTER(C.c_uint8)),
                         types=C.cast(t, C.POINTER(lib.TypeDesc)), dtype=dtype,
                         softmax_scale=0.0, workspace=None, workspace_bytes=0, stream=None)
        mask = C.c_uint32(0)
        ptrs = (C.c_void_p * 1)()
        st = lib.load().pab_step_dispatch(C.byref(d), 0, C.byref(mask), ptrs)
        assert st == code, (dtype, missing, st)


def test_dispatch_module_rejects_slot_scratch_overlap():
    sched = np.ones((2, 1), dtype=np.uint8)
    t = (lib.TypeDesc * 1)()
    t[0].kind = lib.KINDS["temporal"]
    t[0].B, t[0].H, t[0].F, t[0].S, t[0].D = 1, 2, 2, 8, 64
    t[0].slot[0], t[0].slot[1] = 0x100000, 0x200000
    t[0].x, t[0].w_in, t[0].w_out = 0x300000, 0x400000, 0x500000
    for j in range(4):
        t[0].scratch[j] = 0x600000 + j * 0x100000
    t[0].scratch[3] = 0x200000 + 64   # inside slot[1]
    d = lib.StepDesc(num_steps=2, num_types=1,
                     recompute=sched.ctypes.data_as(C.POINTER(C.c_uint8)),
                     types=C.cast(t, C.POINTER(lib.TypeDesc)), dtype=lib.PAB_BF16,
                     softmax_scale=0.0, workspace=None, workspace_bytes=0, stream=None)
    mask = C.c_uint32(0)
    ptrs = (C.c_void_p * 1)()
    assert lib.load().pab_step_dispatch(C.byref(d), 0, C.byref(mask), ptrs) == lib.PAB_ERR_INVALID_ARG


def test_projection_validation_codes():
    # pab_proj_in / pab_proj_out: bf16 only, C = H*D a multiple of 32,
    # 1..3 outputs, no aliasing; checked on the host before any launch.
    L = lib.load()
    pin, pout = L.pab_proj_in, L.pab_proj_out
    X, W, Y0, Y1, Y2 = (C.c_void_p(a) for a in (0x1000000, 0x2000000, 0x3000000, 0x4000000,
                                                 0x5000000))
    ok_args = (1, 2, 10, 4, 64)  # B, F, S, H, D  (C = 256)
    assert pin(X, W, Y0, Y1, Y2, 0, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pin(X, W, Y0, Y1, Y2, 4, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pin(X, W, Y0, None, Y2, 3, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pin(X, W, Y0, Y1, Y2, 3, *ok_args, lib.PAB_F32, None) == lib.PAB_ERR_UNSUPPORTED
    assert pin(X, W, Y0, Y1, Y2, 3, 1, 2, 10, 3, 40, lib.PAB_BF16, None) == lib.PAB_ERR_UNSUPPORTED
    assert "multiple of 32" in lib.pab_last_error()
    assert pin(X, W, Y0, Y0, Y2, 3, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pin(X, W, X, Y1, Y2, 3, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pin(C.c_void_p(0x1000008), W, Y0, Y1, Y2, 3, *ok_args, lib.PAB_BF16, None) == \
        lib.PAB_ERR_INVALID_ARG
    assert pin(X, W, Y0, Y1, Y2, 3, 0, 2, 10, 4, 64, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pout(X, W, None, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pout(X, W, X, *ok_args, lib.PAB_BF16, None) == lib.PAB_ERR_INVALID_ARG
    assert pout(X, W, Y0, *ok_args, lib.PAB_F32, None) == lib.PAB_ERR_UNSUPPORTED
    assert pout(X, W, Y0, 1, 2, 10, 4, 60, lib.PAB_BF16, None) == lib.PAB_ERR_UNSUPPORTED
