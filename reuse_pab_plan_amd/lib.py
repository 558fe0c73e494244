"""ctypes binding of libpab.so (declared in include/pab.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name; all computation happens in the library's HIP kernels.
Device tensors are torch tensors (torch provides device memory and streams).
If the library is missing this module raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpab.so")

PAB_OK = 0
PAB_ERR_INVALID_ARG = -1
PAB_ERR_UNSUPPORTED = -2
PAB_ERR_DEVICE = -3
PAB_ERR_CAPACITY = -4

PAB_BF16 = 0
PAB_F32 = 1

PAB_SPATIAL = 0
PAB_TEMPORAL = 1
PAB_CROSS = 2
KINDS = {"spatial": PAB_SPATIAL, "temporal": PAB_TEMPORAL, "cross": PAB_CROSS}

# Every symbol include/pab.h declares.
EXPORTED = (
    "pab_plan_schedule",
    "pab_plan_calibrate",
    "pab_attn_spatial",
    "pab_attn_temporal",
    "pab_attn_cross",
    "pab_attn_cross_masked",
    "pab_proj_in",
    "pab_proj_out",
    "pab_mse_workspace_bytes",
    "pab_attn_diff_mse",
    "pab_step_dispatch",
    "pab_last_error",
    "pab_version",
)

# Measurement helpers (include/pab_peaks.h): microbenchmarks for the roofline
# denominators, not part of the method.
EXPORTED_PEAKS = (
    "pab_peak_sink_bytes",
    "pab_peak_copy",
    "pab_peak_read",
    "pab_peak_mfma_bf16",
    "pab_peak_exp",
)


class PabError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class TypeDesc(C.Structure):
    _fields_ = [
        ("kind", C.c_int32),
        ("q", C.c_void_p),
        ("k", C.c_void_p),
        ("v", C.c_void_p),
        ("slot", C.c_void_p * 2),
        ("B", C.c_int32),
        ("H", C.c_int32),
        ("F", C.c_int32),
        ("S", C.c_int32),
        ("D", C.c_int32),
        ("L", C.c_int32),
        ("drift", C.c_void_p),
        ("text_len", C.POINTER(C.c_int32)),
        ("x", C.c_void_p),
        ("x_text", C.c_void_p),
        ("w_in", C.c_void_p),
        ("w_kv", C.c_void_p),
        ("w_out", C.c_void_p),
        ("scratch", C.c_void_p * 4),
    ]


class StepDesc(C.Structure):
    _fields_ = [
        ("num_steps", C.c_int32),
        ("num_types", C.c_int32),
        ("recompute", C.POINTER(C.c_uint8)),
        ("types", C.POINTER(TypeDesc)),
        ("dtype", C.c_int32),
        ("softmax_scale", C.c_float),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
        ("stream", C.c_void_p),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Open libpab.so once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m reuse_pab_plan_amd.build` "
            "(the PAB path has no non-HIP fallback)"
        )
    lib = C.CDLL(path)
    i32, i64, f32, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
    lib.pab_plan_schedule.argtypes = [i32, i32, C.POINTER(i32), i32, i32,
                                      C.POINTER(C.c_uint8), C.POINTER(i32), C.POINTER(i32)]
    lib.pab_plan_schedule.restype = C.c_int
    lib.pab_plan_calibrate.argtypes = [i32, i32, C.POINTER(C.c_double), i32, i32,
                                       C.POINTER(i32), C.POINTER(i32), C.POINTER(C.c_double)]
    lib.pab_plan_calibrate.restype = C.c_int
    for name in ("pab_attn_spatial", "pab_attn_temporal"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
        fn.restype = C.c_int
    lib.pab_attn_cross.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp]
    lib.pab_attn_cross.restype = C.c_int
    lib.pab_attn_cross_masked.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32,
                                          C.POINTER(i32), vp]
    lib.pab_attn_cross_masked.restype = C.c_int
    lib.pab_proj_in.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pab_proj_in.restype = C.c_int
    lib.pab_proj_out.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pab_proj_out.restype = C.c_int
    lib.pab_mse_workspace_bytes.argtypes = [i64]
    lib.pab_mse_workspace_bytes.restype = sz
    lib.pab_attn_diff_mse.argtypes = [vp, vp, i64, i32, vp, vp, sz, vp]
    lib.pab_attn_diff_mse.restype = C.c_int
    lib.pab_step_dispatch.argtypes = [C.POINTER(StepDesc), i32, C.POINTER(C.c_uint32),
                                      C.POINTER(C.c_void_p)]
    lib.pab_step_dispatch.restype = C.c_int
    lib.pab_last_error.argtypes = []
    lib.pab_last_error.restype = C.c_char_p
    lib.pab_version.argtypes = []
    lib.pab_version.restype = C.c_char_p
    lib.pab_peak_sink_bytes.argtypes = []
    lib.pab_peak_sink_bytes.restype = sz
    lib.pab_peak_copy.argtypes = [vp, vp, sz, vp]
    lib.pab_peak_copy.restype = C.c_int
    lib.pab_peak_read.argtypes = [vp, sz, vp, sz, vp]
    lib.pab_peak_read.restype = C.c_int
    for name in ("pab_peak_mfma_bf16", "pab_peak_exp"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, vp, sz, C.POINTER(C.c_double), vp]
        fn.restype = C.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != PAB_OK:
        raise PabError(fn, status, load().pab_last_error().decode())


def pab_last_error() -> str:
    return load().pab_last_error().decode()


def pab_version() -> str:
    return load().pab_version().decode()


# ------------------------------------------------------------------ host side

def pab_plan_schedule(num_steps: int, ranges, window_lo_pct: int = 15, window_hi_pct: int = 85):
    """Returns (recompute uint8 [N,T], source_step int32 [N,T], counts int32 [T])."""
    lib = load()
    t = len(ranges)
    r = np.ascontiguousarray(np.asarray(ranges, dtype=np.int32))
    rec = np.zeros((max(num_steps, 0), t), dtype=np.uint8)
    src = np.zeros((max(num_steps, 0), t), dtype=np.int32)
    cnt = np.zeros(t, dtype=np.int32)
    st = lib.pab_plan_schedule(
        num_steps, t, r.ctypes.data_as(C.POINTER(C.c_int32)), window_lo_pct, window_hi_pct,
        rec.ctypes.data_as(C.POINTER(C.c_uint8)), src.ctypes.data_as(C.POINTER(C.c_int32)),
        cnt.ctypes.data_as(C.POINTER(C.c_int32)),
    )
    _check("pab_plan_schedule", st)
    return rec, src, cnt


def pab_plan_calibrate(diff, candidate_ranges, window_lo_pct: int = 15, window_hi_pct: int = 85):
    """diff: [N, T] attention differences (row i: steps i-1 -> i).
    Returns (ranges int32 [T], scores float64 [T])."""
    lib = load()
    d = np.ascontiguousarray(np.asarray(diff, dtype=np.float64))
    n, t = d.shape
    c = np.ascontiguousarray(np.asarray(candidate_ranges, dtype=np.int32))
    if c.shape != (t,):
        raise ValueError("one candidate range per attention type")
    out = np.zeros(t, dtype=np.int32)
    sc = np.zeros(t, dtype=np.float64)
    st = lib.pab_plan_calibrate(
        n, t, d.ctypes.data_as(C.POINTER(C.c_double)), window_lo_pct, window_hi_pct,
        c.ctypes.data_as(C.POINTER(C.c_int32)), out.ctypes.data_as(C.POINTER(C.c_int32)),
        sc.ctypes.data_as(C.POINTER(C.c_double)))
    _check("pab_plan_calibrate", st)
    return out, sc


# ---------------------------------------------------------------- device side

def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return PAB_BF16
    if t.dtype == torch.float32:
        return PAB_F32
    raise PabError("binding", PAB_ERR_UNSUPPORTED, f"dtype {t.dtype} unsupported")


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def pab_attn_spatial(q, k, v, o, softmax_scale: float = 0.0, stream=None):
    """q, k, v, o: [B, H, F, S, D] device tensors (bf16 or fp32)."""
    B, H, F, S, D = q.shape
    st = load().pab_attn_spatial(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, F, S, D,
                                 _dtype_code(q), softmax_scale, _stream_ptr(stream))
    _check("pab_attn_spatial", st)
    return o


def pab_attn_temporal(q, k, v, o, softmax_scale: float = 0.0, stream=None):
    """q, k, v, o: [B, H, F, S, D] device tensors (bf16 or fp32)."""
    B, H, F, S, D = q.shape
    st = load().pab_attn_temporal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, F, S, D,
                                  _dtype_code(q), softmax_scale, _stream_ptr(stream))
    _check("pab_attn_temporal", st)
    return o


def pab_attn_cross(q, k_text, v_text, o, softmax_scale: float = 0.0, stream=None):
    """q, o: [B, H, ..., D] video queries; k_text, v_text: [B, H, L, D]."""
    B, H = q.shape[0], q.shape[1]
    D = q.shape[-1]
    nq = q.numel() // (B * H * D)
    L = k_text.shape[2]
    st = load().pab_attn_cross(_ptr(q), _ptr(k_text), _ptr(v_text), _ptr(o), B, H, nq, L, D,
                               _dtype_code(q), softmax_scale, _stream_ptr(stream))
    _check("pab_attn_cross", st)
    return o


def pab_attn_cross_masked(q, k_text, v_text, o, text_len, softmax_scale: float = 0.0, stream=None):
    """As pab_attn_cross; batch entry b attends to its first text_len[b] text tokens."""
    B, H = q.shape[0], q.shape[1]
    D = q.shape[-1]
    nq = q.numel() // (B * H * D)
    L = k_text.shape[2]
    lens = np.ascontiguousarray(np.asarray(text_len, dtype=np.int32))
    if lens.shape != (B,):
        raise ValueError("one text length per batch entry")
    st = load().pab_attn_cross_masked(_ptr(q), _ptr(k_text), _ptr(v_text), _ptr(o), B, H, nq, L, D,
                                      _dtype_code(q), softmax_scale,
                                      lens.ctypes.data_as(C.POINTER(C.c_int32)), _stream_ptr(stream))
    _check("pab_attn_cross_masked", st)
    return o


def pab_proj_in(x, w, outs, frames: int, tokens: int, heads: int, head_dim: int, stream=None):
    """x: [B, F*S, C] token-major; w: [n*C, C]; outs: n head-major tensors [B, H, F, S, D]."""
    n = len(outs)
    ptrs = [_ptr(t) for t in outs] + [None] * (3 - n)
    st = load().pab_proj_in(_ptr(x), _ptr(w), ptrs[0], ptrs[1], ptrs[2], n, x.shape[0], frames,
                            tokens, heads, head_dim, _dtype_code(x), _stream_ptr(stream))
    _check("pab_proj_in", st)
    return outs


def pab_proj_out(o, w, y, stream=None):
    """o: [B, H, F, S, D] head-major; w: [C, C]; y: [B, F*S, C] token-major."""
    B, H, F, S, D = o.shape
    st = load().pab_proj_out(_ptr(o), _ptr(w), _ptr(y), B, F, S, H, D, _dtype_code(o),
                             _stream_ptr(stream))
    _check("pab_proj_out", st)
    return y


def pab_mse_workspace_bytes(n: int) -> int:
    return int(load().pab_mse_workspace_bytes(n))


def pab_attn_diff_mse(a, b, out, workspace, stream=None):
    """out: 1-element float64 device tensor; workspace: device buffer (uint8)."""
    n = a.numel()
    st = load().pab_attn_diff_mse(_ptr(a), _ptr(b), n, _dtype_code(a), _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check("pab_attn_diff_mse", st)
    return out


def pab_step_dispatch(desc: StepDesc, step: int):
    """Returns (recomputed_mask, [output pointer per type])."""
    mask = C.c_uint32(0)
    outs = (C.c_void_p * desc.num_types)()
    st = load().pab_step_dispatch(C.byref(desc), step, C.byref(mask), outs)
    _check("pab_step_dispatch", st)
    return mask.value, [outs[a] for a in range(desc.num_types)]


# ------------------------------------------------------------ measurement aids

def measure_peaks(device=None, stream=None):
    """Sustained peaks of this GPU from the pab_peak_* microbenchmarks, each
    the best of a few launches timed with HIP events on ``stream``: HBM copy
    (read + write) and read in GB/s over buffers rotated past the 256 MB
    Infinity Cache, bf16 MFMA in TFLOP/s, v_exp_f32 in G/s."""
    import torch

    L = load()
    dev = device or torch.device("cuda:0")
    st = stream or torch.cuda.current_stream(dev)
    sp = C.c_void_p(st.cuda_stream)
    sink = torch.empty(int(L.pab_peak_sink_bytes()), dtype=torch.uint8, device=dev)
    nbuf, nbytes = 4, 256 << 20
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2 * nbuf)]
    for b in bufs:
        b.fill_(1)

    def best(launch, n=6):
        ts = []
        for i in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            launch(i)
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts[1:])

    out = {}
    t = best(lambda i: _check("pab_peak_copy", L.pab_peak_copy(
        C.c_void_p(bufs[i % nbuf].data_ptr()), C.c_void_p(bufs[nbuf + i % nbuf].data_ptr()),
        nbytes, sp)))
    out["hbm_copy_gbs"] = 2 * nbytes / t / 1e9
    t = best(lambda i: _check("pab_peak_read", L.pab_peak_read(
        C.c_void_p(bufs[i % (2 * nbuf)].data_ptr()), nbytes, C.c_void_p(sink.data_ptr()),
        sink.numel(), sp)))
    out["hbm_read_gbs"] = nbytes / t / 1e9
    work = C.c_double(0.0)
    t = best(lambda i: _check("pab_peak_mfma_bf16", L.pab_peak_mfma_bf16(
        2048, C.c_void_p(sink.data_ptr()), sink.numel(), C.byref(work), sp)))
    out["mfma_bf16_tflops"] = work.value / t / 1e12
    t = best(lambda i: _check("pab_peak_exp", L.pab_peak_exp(
        2048, C.c_void_p(sink.data_ptr()), sink.numel(), C.byref(work), sp)))
    out["exp_gps"] = work.value / t / 1e9
    del bufs, sink
    torch.cuda.empty_cache()
    return out
