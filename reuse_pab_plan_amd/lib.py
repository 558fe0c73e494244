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
# PAB_LIB may name another build of the same library (e.g. the host-side
# sanitizer build, libpab_san.so).
LIB_PATH = os.environ.get("PAB_LIB") or os.path.join(_HERE, "libpab.so")

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
    "pab_attn_diff_mse_noalloc",
    "pab_step_dispatch",
    "pab_last_error",
    "pab_version",
)

# Measurement helpers (include/pab_peaks.h): microbenchmarks for the roofline
# denominators, not part of the method.
EXPORTED_PEAKS = (
    "pab_peak_sink_bytes",
    "pab_peak_stream",
    "pab_peak_mfma_bf16",
    "pab_peak_exp",
)

# Workload generator (include/pab_synth.h): seeded synthetic inputs, not part
# of the method.
EXPORTED_SYNTH = (
    "pab_synth_philox",
    "pab_synth_normal",
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
    lib.pab_plan_calibrate.argtypes = [i32, i32, i32, C.POINTER(C.c_double), i32, i32,
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
    lib.pab_attn_diff_mse_noalloc.argtypes = [vp, vp, i64, i32, vp, vp]
    lib.pab_attn_diff_mse_noalloc.restype = C.c_int
    lib.pab_step_dispatch.argtypes = [C.POINTER(StepDesc), i32, C.POINTER(C.c_uint32),
                                      C.POINTER(C.c_void_p)]
    lib.pab_step_dispatch.restype = C.c_int
    lib.pab_last_error.argtypes = []
    lib.pab_last_error.restype = C.c_char_p
    lib.pab_version.argtypes = []
    lib.pab_version.restype = C.c_char_p
    lib.pab_synth_philox.argtypes = [vp, i64, C.c_uint64, C.c_uint64, vp]
    lib.pab_synth_philox.restype = C.c_int
    lib.pab_synth_normal.argtypes = [vp, i64, i32, C.c_uint64, f32, C.c_uint64, f32, vp]
    lib.pab_synth_normal.restype = C.c_int
    lib.pab_peak_sink_bytes.argtypes = []
    lib.pab_peak_sink_bytes.restype = sz
    lib.pab_peak_stream.argtypes = [C.POINTER(vp), i32, C.POINTER(vp), i32, sz, i32, i32, vp, sz,
                                    vp]
    lib.pab_peak_stream.restype = C.c_int
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
    """diff: [N, T] attention differences of one block (row i: steps i-1 ->
    i), or [blocks, N, T] for a stack sharing one schedule.
    Returns (ranges int32 [T], scores float64 [T])."""
    lib = load()
    d = np.ascontiguousarray(np.asarray(diff, dtype=np.float64))
    if d.ndim == 2:
        d = d[None]
    if d.ndim != 3:
        raise ValueError("diff must be [N, T] or [blocks, N, T]")
    nb, n, t = d.shape
    c = np.ascontiguousarray(np.asarray(candidate_ranges, dtype=np.int32))
    if c.shape != (t,):
        raise ValueError("one candidate range per attention type")
    out = np.zeros(t, dtype=np.int32)
    sc = np.zeros(t, dtype=np.float64)
    st = lib.pab_plan_calibrate(
        nb, n, t, d.ctypes.data_as(C.POINTER(C.c_double)), window_lo_pct, window_hi_pct,
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


def _bad(fn, msg):
    raise PabError(fn, PAB_ERR_INVALID_ARG, msg)


def _dense(fn, **tensors):
    """Each tensor must be contiguous (the library takes a bare pointer and
    assumes the documented dense layout) and on the GPU."""
    for name, t in tensors.items():
        if t is None:
            _bad(fn, f"{name} is None")
        if not t.is_contiguous():
            _bad(fn, f"{name} must be contiguous (a strided view would be read as dense)")
    for name, t in tensors.items():
        if not t.is_cuda:
            _bad(fn, f"{name} must be a device tensor")


def _same(fn, ref_name, ref, **tensors):
    """Every tensor has the reference's shape and dtype."""
    for name, t in tensors.items():
        if tuple(t.shape) != tuple(ref.shape):
            _bad(fn, f"{name} has shape {tuple(t.shape)}, {ref_name} {tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            _bad(fn, f"{name} has dtype {t.dtype}, {ref_name} {ref.dtype}")


def _video_attn_args(fn, q, k, v, o):
    if q.dim() != 5:
        _bad(fn, f"q must be [B, H, F, S, D], got {tuple(q.shape)}")
    _same(fn, "q", q, k=k, v=v, o=o)
    _dense(fn, q=q, k=k, v=v, o=o)


def _cross_args(fn, q, k_text, v_text, o):
    if q.dim() < 3:
        _bad(fn, f"q must be [B, H, ..., D], got {tuple(q.shape)}")
    _same(fn, "q", q, o=o)
    _same(fn, "k_text", k_text, v_text=v_text)
    B, H, D = q.shape[0], q.shape[1], q.shape[-1]
    if k_text.dim() != 4 or (k_text.shape[0], k_text.shape[1], k_text.shape[3]) != (B, H, D):
        _bad(fn, f"k_text must be [B, H, L, D] = [{B}, {H}, L, {D}], got {tuple(k_text.shape)}")
    if k_text.dtype != q.dtype:
        _bad(fn, f"k_text has dtype {k_text.dtype}, q {q.dtype}")
    _dense(fn, q=q, k_text=k_text, v_text=v_text, o=o)


def pab_attn_spatial(q, k, v, o, softmax_scale: float = 0.0, stream=None):
    """q, k, v, o: [B, H, F, S, D] device tensors (bf16 or fp32)."""
    _video_attn_args("pab_attn_spatial", q, k, v, o)
    B, H, F, S, D = q.shape
    st = load().pab_attn_spatial(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, F, S, D,
                                 _dtype_code(q), softmax_scale, _stream_ptr(stream))
    _check("pab_attn_spatial", st)
    return o


def pab_attn_temporal(q, k, v, o, softmax_scale: float = 0.0, stream=None):
    """q, k, v, o: [B, H, F, S, D] device tensors (bf16 or fp32)."""
    _video_attn_args("pab_attn_temporal", q, k, v, o)
    B, H, F, S, D = q.shape
    st = load().pab_attn_temporal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, F, S, D,
                                  _dtype_code(q), softmax_scale, _stream_ptr(stream))
    _check("pab_attn_temporal", st)
    return o


def pab_attn_cross(q, k_text, v_text, o, softmax_scale: float = 0.0, stream=None):
    """q, o: [B, H, ..., D] video queries; k_text, v_text: [B, H, L, D]."""
    _cross_args("pab_attn_cross", q, k_text, v_text, o)
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
    _cross_args("pab_attn_cross_masked", q, k_text, v_text, o)
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
    fn = "pab_proj_in"
    n = len(outs)
    if not 1 <= n <= 3:
        _bad(fn, "one to three output tensors")
    C_ = heads * head_dim
    if x.dim() != 3 or x.shape[1] != frames * tokens or x.shape[2] != C_:
        _bad(fn, f"x must be [B, F*S, H*D] = [B, {frames * tokens}, {C_}], got {tuple(x.shape)}")
    if tuple(w.shape) != (n * C_, C_):
        _bad(fn, f"w must be [{n * C_}, {C_}], got {tuple(w.shape)}")
    want = x.shape[0] * heads * frames * tokens * head_dim
    for j, t in enumerate(outs):
        if t.numel() != want or t.dtype != x.dtype:
            _bad(fn, f"out{j} must hold {want} elements of {x.dtype}")
    if w.dtype != x.dtype:
        _bad(fn, f"w has dtype {w.dtype}, x {x.dtype}")
    _dense(fn, x=x, w=w, **{f"out{j}": t for j, t in enumerate(outs)})
    ptrs = [_ptr(t) for t in outs] + [None] * (3 - n)
    st = load().pab_proj_in(_ptr(x), _ptr(w), ptrs[0], ptrs[1], ptrs[2], n, x.shape[0], frames,
                            tokens, heads, head_dim, _dtype_code(x), _stream_ptr(stream))
    _check("pab_proj_in", st)
    return outs


def pab_proj_out(o, w, y, stream=None):
    """o: [B, H, F, S, D] head-major; w: [C, C]; y: [B, F*S, C] token-major."""
    fn = "pab_proj_out"
    if o.dim() != 5:
        _bad(fn, f"o must be [B, H, F, S, D], got {tuple(o.shape)}")
    B, H, F, S, D = o.shape
    if tuple(w.shape) != (H * D, H * D) or w.dtype != o.dtype:
        _bad(fn, f"w must be [{H * D}, {H * D}] of {o.dtype}")
    if y.numel() != o.numel() or y.dtype != o.dtype:
        _bad(fn, f"y must hold {o.numel()} elements of {o.dtype}")
    _dense(fn, o=o, w=w, y=y)
    st = load().pab_proj_out(_ptr(o), _ptr(w), _ptr(y), B, F, S, H, D, _dtype_code(o),
                             _stream_ptr(stream))
    _check("pab_proj_out", st)
    return y


def pab_mse_workspace_bytes(n: int) -> int:
    return int(load().pab_mse_workspace_bytes(n))


def pab_attn_diff_mse(a, b, out, workspace, stream=None):
    """out: 1-element float64 device tensor; workspace: device buffer (uint8)."""
    import torch

    fn = "pab_attn_diff_mse"
    if a.numel() != b.numel() or a.dtype != b.dtype:
        _bad(fn, "a and b must have the same number of elements and dtype")
    if out.dtype != torch.float64 or out.numel() < 1:
        _bad(fn, "out must be a float64 tensor of at least one element")
    _dense(fn, a=a, b=b, out=out, workspace=workspace)
    n = a.numel()
    st = load().pab_attn_diff_mse(_ptr(a), _ptr(b), n, _dtype_code(a), _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check("pab_attn_diff_mse", st)
    return out


def pab_attn_diff_mse_noalloc(a, b, out, stream=None):
    """As pab_attn_diff_mse, with the library's own device scratch (no
    workspace, no allocation)."""
    import torch

    fn = "pab_attn_diff_mse_noalloc"
    if a.numel() != b.numel() or a.dtype != b.dtype:
        _bad(fn, "a and b must have the same number of elements and dtype")
    if out.dtype != torch.float64 or out.numel() < 1:
        _bad(fn, "out must be a float64 tensor of at least one element")
    _dense(fn, a=a, b=b, out=out)
    st = load().pab_attn_diff_mse_noalloc(_ptr(a), _ptr(b), a.numel(), _dtype_code(a), _ptr(out),
                                          _stream_ptr(stream))
    _check(fn, st)
    return out


def pab_step_dispatch(desc: StepDesc, step: int):
    """Returns (recomputed_mask, [output pointer per type])."""
    mask = C.c_uint32(0)
    outs = (C.c_void_p * desc.num_types)()
    st = load().pab_step_dispatch(C.byref(desc), step, C.byref(mask), outs)
    _check("pab_step_dispatch", st)
    return mask.value, [outs[a] for a in range(desc.num_types)]


# ---------------------------------------------------------- workload generator

def pab_synth_philox(out, key: int, block0: int = 0, stream=None):
    """out: int32 device tensor of 4*nblocks elements (the uint32 words, as
    bits): words of Philox4x32-10 blocks block0.. of stream ``key``."""
    fn = "pab_synth_philox"
    if out.element_size() != 4 or out.numel() % 4:
        _bad(fn, "out must hold a multiple of four 32-bit words")
    _dense(fn, out=out)
    st = load().pab_synth_philox(_ptr(out), out.numel() // 4, key, block0, _stream_ptr(stream))
    _check(fn, st)
    return out


def pab_synth_normal(out, key_a: int, scale_a: float, key_b: int = 0, scale_b: float = 0.0,
                     stream=None):
    """out (bf16 or fp32 device tensor) = round(scale_a N(key_a) + scale_b N(key_b))."""
    fn = "pab_synth_normal"
    _dense(fn, out=out)
    st = load().pab_synth_normal(_ptr(out), out.numel(), _dtype_code(out), key_a, scale_a, key_b,
                                 scale_b, _stream_ptr(stream))
    _check(fn, st)
    return out


# ------------------------------------------------------------ measurement aids

def cache_scrub(buf, sink, stream=None):
    """Read ``buf`` (device, uint8, much larger than the 256 MB Infinity Cache)
    once with the streaming microbenchmark: dirty lines left by earlier
    writes are written back and the caches hold clean, unrelated data."""
    L = load()
    src = (C.c_void_p * 1)(buf.data_ptr())
    dst = (C.c_void_p * 1)()
    _check("pab_peak_stream", L.pab_peak_stream(src, 1, dst, 0, buf.numel(), 8192, 1,
                                                 C.c_void_p(sink.data_ptr()), sink.numel(),
                                                 _stream_ptr(stream)))


# Read:write stream mixes measured by measure_peaks: name -> (sources,
# destinations).  The attention kernels' own mixes: temporal reads Q, K, V
# (and the previous output when it takes the attention difference) and
# writes O; cross reads Q (and the previous output) and writes O (its text
# K/V are negligible); the MSE reads two tensors.
STREAM_MIXES = {"1:0": (1, 0), "0:1": (0, 1), "1:1": (1, 1), "2:1": (2, 1), "3:1": (3, 1),
                "4:1": (4, 1), "2:0": (2, 0)}


def measure_peaks(device=None, stream=None, stream_bytes=1 << 30):
    """Sustained peaks of this GPU from the pab_peak_* microbenchmarks.

    HBM: for every read:write mix in STREAM_MIXES, the best rate
    ((sources + destinations) x stream_bytes per launch, 1 GiB streams by
    default, two buffer sets used alternately) over grids of 1024 to 16384
    blocks, plain or non-temporal accesses, 4, 8 or 16 vectors in flight per
    stream and thread, grid-stride or block-contiguous walks, each timed
    with HIP events on ``stream``; bf16 MFMA in TFLOP/s and v_exp_f32 in G/s
    (best of a few launches).
    """
    import torch

    L = load()
    dev = device or torch.device("cuda:0")
    st = stream or torch.cuda.current_stream(dev)
    sp = C.c_void_p(st.cuda_stream)
    sink = torch.empty(int(L.pab_peak_sink_bytes()), dtype=torch.uint8, device=dev)
    sets = [[torch.empty(stream_bytes, dtype=torch.uint8, device=dev) for _ in range(6)]
            for _ in range(2)]
    for bs in sets:
        for b in bs:
            b.fill_(1)

    def timed(launch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        launch()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    out = {"hbm_stream_gbs": {}, "hbm_stream_best": {}, "stream_bytes": stream_bytes}
    k = 0
    for name, (ns, nd) in STREAM_MIXES.items():
        best, how = None, None
        for blocks in (1024, 2048, 4096, 8192, 16384):
            for variant in (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13):
                for rep in range(2):
                    bs = sets[k % 2]
                    k += 1
                    src = (C.c_void_p * 4)(*[b.data_ptr() for b in bs[:4]])
                    dst = (C.c_void_p * 2)(*[b.data_ptr() for b in bs[4:6]])
                    t = timed(lambda: _check("pab_peak_stream", L.pab_peak_stream(
                        src, ns, dst, nd, stream_bytes, blocks, variant,
                        C.c_void_p(sink.data_ptr()), sink.numel(), sp)))
                    if rep and (best is None or t < best):
                        best, how = t, {"blocks": blocks, "non_temporal": bool(variant & 1),
                                        "in_flight": 4 << ((variant >> 1) & 3),
                                        "contiguous_blocks": bool(variant & 8)}
        out["hbm_stream_gbs"][name] = (ns + nd) * stream_bytes / best / 1e9
        out["hbm_stream_best"][name] = how
    out["hbm_read_gbs"] = out["hbm_stream_gbs"]["1:0"]
    out["hbm_write_gbs"] = out["hbm_stream_gbs"]["0:1"]
    out["hbm_copy_gbs"] = out["hbm_stream_gbs"]["1:1"]
    del sets

    def best_of(launch, n=6):
        return min(timed(launch) for _ in range(n))

    work = C.c_double(0.0)
    t = best_of(lambda: _check("pab_peak_mfma_bf16", L.pab_peak_mfma_bf16(
        2048, C.c_void_p(sink.data_ptr()), sink.numel(), C.byref(work), sp)))
    out["mfma_bf16_tflops"] = work.value / t / 1e12
    t = best_of(lambda: _check("pab_peak_exp", L.pab_peak_exp(
        2048, C.c_void_p(sink.data_ptr()), sink.numel(), C.byref(work), sp)))
    out["exp_gps"] = work.value / t / 1e9
    del sink
    torch.cuda.empty_cache()
    return out
