"""Trajectory harness: runs a denoising trajectory of one or more DiT blocks
through libpab.so's broadcast schedule and step dispatcher.

PAB article, Figure 2 caption: each step either computes an attention type or
reuses the output broadcast from an earlier step.  The harness plans the
schedule with ``pab_plan_schedule``, allocates the cache slots (two O-sized
HBM buffers per block and type), and for every step calls
``pab_step_dispatch`` once per attention type, bracketed by HIP events on the
launch stream; with drift on, the dispatcher also takes the attention
difference (MSE) between each recompute and the output it replaces (PAB
article, Figure 1 caption).  torch supplies device memory, streams and
events only.

``CONFIGS`` holds the synthetic workloads, stand-ins for the video DiTs the
pages measure (480p and 720p latent shapes, a 28-block stack, a full-3D
attention model); their inputs come from ``synth``.
"""

from __future__ import annotations

import ctypes as C
import dataclasses

import numpy as np

from . import lib, synth


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str          # "bf16" or "f32"
    B: int
    H: int
    F: int
    S: int
    D: int
    L: int
    N: int              # denoising steps
    kinds: tuple        # attention types of one block
    ranges: tuple       # broadcast range per type
    blocks: int
    seed: int
    desc: str
    # Real text tokens per batch entry (padded prompts; None = all L real),
    # and whether the text K/V stay the same at every step (as a real text
    # encoder's would) instead of following the perturbation model.
    text_len: tuple | None = None
    const_text: bool = False
    # Whole attention modules: each recompute runs the input projection, the
    # attention and the output projection; a broadcast step skips all three.
    module: bool = False

    @property
    def C(self):
        return self.H * self.D

    @property
    def video_shape(self):
        return (self.B, self.H, self.F, self.S, self.D)

    @property
    def text_shape(self):
        return (self.B, self.H, self.L, self.D)

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4


CONFIGS = {
    "tiny": Config("tiny", "f32", 1, 4, 4, 64, 64, 16, 10, ("spatial", "temporal", "cross"),
                   (2, 3, 5), 1, 1,
                   "tiny fp32: 4 frames x 64 tokens, 4 heads x 64, 16 text tokens, 10 steps"),
    "b480": Config("b480", "bf16", 1, 16, 48, 1590, 72, 120, 30, ("spatial", "temporal", "cross"),
                   (2, 4, 6), 1, 2,
                   "480p-latent block: 48 frames x 1590 tokens, 16 heads x 72, 120 text tokens, 30 steps"),
    "b720": Config("b720", "bf16", 1, 16, 32, 3600, 72, 120, 30, ("spatial", "temporal", "cross"),
                   (2, 4, 6), 1, 3,
                   "720p-latent block: 32 frames x 3600 tokens, 16 heads x 72, 120 text tokens, 30 steps"),
    "stack28": Config("stack28", "bf16", 1, 16, 48, 1590, 72, 120, 30,
                      ("spatial", "temporal", "cross"), (2, 4, 6), 28, 4,
                      "28-block stack at the 480p-latent shape, 30 steps"),
    "full3d": Config("full3d", "bf16", 2, 24, 1, 16384, 64, 120, 50, ("spatial", "cross"), (2, 6),
                     1, 5, "full-3D attention, CFG batch 2: 16384 tokens, 24 heads x 64, 120 text "
                     "tokens, 50 steps"),
    # Padded prompts with classifier-free guidance: the conditional entry has
    # 77 real text tokens of 120, the unconditional (empty prompt) one; text
    # K/V constant over the steps.
    "cfg480": Config("cfg480", "bf16", 2, 16, 48, 1590, 72, 120, 30,
                     ("spatial", "temporal", "cross"), (2, 4, 6), 1, 6,
                     "480p-latent block, CFG batch 2 with padded prompts (77 and 1 real text "
                     "tokens of 120, constant text K/V), 30 steps",
                     text_len=(77, 1), const_text=True),
    # Attention modules (projections around each attention).
    "mod_small": Config("mod_small", "bf16", 1, 4, 4, 100, 64, 16, 10,
                        ("spatial", "temporal", "cross"), (2, 3, 5), 1, 7,
                        "attention modules: 4 frames x 100 tokens, 4 heads x 64 (C = 256), "
                        "16 text tokens, 10 steps", module=True),
    "b480m": Config("b480m", "bf16", 1, 16, 48, 1590, 72, 120, 30,
                    ("spatial", "temporal", "cross"), (2, 4, 6), 1, 8,
                    "480p-latent block as attention modules (C = 1152 projections around each "
                    "attention), 30 steps", module=True),
}

TYPE_INDEX = {"spatial": 0, "temporal": 1, "cross": 2}


# ------------------------------------------------------------ algorithmic work

def attn_flops(cfg: Config, kind: str) -> int:
    """QK^T and PV multiply-adds (2 flops each) of one call; nothing padded
    (padding text tokens are not work)."""
    B, H, F, S, D, L = cfg.B, cfg.H, cfg.F, cfg.S, cfg.D, cfg.L
    if kind == "spatial":
        return 4 * B * H * F * S * S * D
    if kind == "temporal":
        return 4 * B * H * S * F * F * D
    text = sum(cfg.text_len) if cfg.text_len else B * L
    return 4 * H * F * S * text * D


def attn_bytes(cfg: Config, kind: str) -> int:
    """Compulsory HBM bytes of one call: inputs read once, output written once."""
    n = cfg.B * cfg.H * cfg.F * cfg.S * cfg.D * cfg.elem_bytes
    if kind == "cross":
        text = sum(cfg.text_len) if cfg.text_len else cfg.B * cfg.L
        return 2 * n + 2 * cfg.H * text * cfg.D * cfg.elem_bytes
    return 4 * n


def proj_flops(cfg: Config, kind: str) -> int:
    """Multiply-adds (2 flops each) of a module's input and output
    projections: token rows x C x C per projected tensor."""
    C_, tokens = cfg.C, cfg.B * cfg.F * cfg.S
    if kind == "cross":
        return 2 * C_ * C_ * (2 * tokens + 2 * cfg.B * cfg.L)
    return 2 * C_ * C_ * 4 * tokens


def cache_bytes(cfg: Config) -> int:
    """HBM the broadcast cache needs: two output-sized slots per (block, type)."""
    return 2 * cfg.blocks * len(cfg.kinds) * cfg.B * cfg.H * cfg.F * cfg.S * cfg.D * cfg.elem_bytes


def check_capacity(need: int, free: int, what: str) -> None:
    """Raise PAB_ERR_CAPACITY (as lib.PabError) when `need` bytes exceed the
    `free` device bytes, before anything is allocated."""
    if need > free:
        raise lib.PabError(what, lib.PAB_ERR_CAPACITY,
                           f"needs {need / 2**30:.2f} GiB of HBM, {free / 2**30:.2f} GiB free")


def mse_bytes(cfg: Config) -> int:
    return 2 * cfg.B * cfg.H * cfg.F * cfg.S * cfg.D * cfg.elem_bytes


# ------------------------------------------------------------------- inputs

class Inputs:
    """Per (block, type, step) Q/K/V device tensors (module configurations:
    the module input x, plus the text tokens for a cross attention, and fixed
    projection weights per (block, type)), drawn by the device generator.

    resident=True generates every needed step up front (the timed region then
    only reads HBM).  Otherwise tensors are generated on demand into a ring of
    two buffer sets: ``get(..., ahead=next)`` returns a step's tensors and
    also draws the next recompute's into the other set, then reads a 512 MB
    scrub buffer.  A kernel thus reads inputs that are in HBM and not in the
    256 MB Infinity Cache, with no dirty lines of the generator's writes
    left to be written back while it runs -- the state of resident inputs.
    """

    def __init__(self, cfg: Config, steps_needed, device="cuda", resident=True):
        import torch

        self.cfg, self.device, self.resident = cfg, device, resident
        self.tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.store = {}
        self._w = {}
        self._ring = None
        self._ring_key = [None, None]
        self._last = 1
        self._scrub_buf = None
        if resident:
            for (b, a, i) in steps_needed:
                self.store[(b, a, i)] = self._make(b, a, i, None)

    def _shapes(self, a):
        cfg = self.cfg
        kind = cfg.kinds[a]
        if cfg.module:
            x = (cfg.B, cfg.F * cfg.S, cfg.C)
            return (x, (cfg.B, cfg.L, cfg.C)) if kind == "cross" else (x,)
        kv = cfg.text_shape if kind == "cross" else cfg.video_shape
        return cfg.video_shape, kv, kv

    def weights(self, b, a):
        """(w_in, w_kv or None, w_out) of a module configuration."""
        if (b, a) not in self._w:
            cfg = self.cfg
            t = TYPE_INDEX[cfg.kinds[a]]
            cross = cfg.kinds[a] == "cross"
            mk = lambda shape, which: synth.gpu_weight(shape, cfg.seed, b, t, which, cfg.dtype,
                                                       self.device)
            self._w[(b, a)] = (mk(((1 if cross else 3) * cfg.C, cfg.C), 0),
                               mk((2 * cfg.C, cfg.C), 1) if cross else None,
                               mk((cfg.C, cfg.C), 2))
        return self._w[(b, a)]

    def _make(self, b, a, i, out):
        shapes = self._shapes(a)
        t = TYPE_INDEX[self.cfg.kinds[a]]
        res = []
        const = self.cfg.const_text and self.cfg.kinds[a] == "cross"
        # Module inputs use their own generator streams (tensors 3 and 4).
        first = 3 if self.cfg.module else 0
        for tensor, shape in enumerate(shapes, start=first):
            dst = None if out is None else out[tensor - first]
            res.append(synth.gpu_tensor(shape, self.cfg.seed, b, t, tensor, i, self.cfg.N,
                                        self.cfg.dtype, self.device, out=dst,
                                        perturb=not (const and tensor != first)))
        return tuple(res)

    def _ring_views(self, slot, a):
        import torch

        if self._ring is None:
            # Each set: one flat buffer per tensor position, as large as the
            # largest tensor any type puts there.
            sizes = [0, 0, 0]
            for a2 in range(len(self.cfg.kinds)):
                for j, shp in enumerate(self._shapes(a2)):
                    sizes[j] = max(sizes[j], int(np.prod(shp)))
            self._ring = [[torch.empty(n, dtype=self.tdt, device=self.device) if n else None
                           for n in sizes] for _ in range(2)]
        return tuple(self._ring[slot][j][:int(np.prod(shp))].view(shp)
                     for j, shp in enumerate(self._shapes(a)))

    def _scrub(self):
        import torch

        if self._scrub_buf is None:
            self._scrub_buf = torch.ones(512 << 20, dtype=torch.uint8, device=self.device)
            self._scrub_sink = torch.empty(lib.load().pab_peak_sink_bytes(), dtype=torch.uint8,
                                           device=self.device)
        lib.cache_scrub(self._scrub_buf, self._scrub_sink)

    def _gen(self, key, slot):
        b, a, i = key
        self._make(b, a, i, self._ring_views(slot, a))
        self._ring_key[slot] = key

    def get(self, b, a, i, ahead=None):
        """The tensors of (block b, type a, step i); with ``ahead`` = the
        (block, type, step) of the next recompute (streamed inputs only), that
        one is drawn too, into the other buffer set."""
        if self.resident:
            return self.store[(b, a, i)]
        key = (b, a, i)
        if key in self._ring_key:
            slot = self._ring_key.index(key)
        else:
            slot = 1 - self._last
            self._gen(key, slot)
        if ahead is not None and ahead not in self._ring_key and ahead != key:
            self._gen(ahead, 1 - slot)
            self._scrub()
        self._last = slot
        return self._ring_views(slot, a)


# --------------------------------------------------------------- trajectory

class Trajectory:
    """One PAB (or PAB-off) trajectory over ``cfg.blocks`` blocks."""

    def __init__(self, cfg: Config, pab: bool = True, inputs: Inputs | None = None,
                 device="cuda", drift: bool = True, stream=None):
        import torch

        self.cfg, self.pab, self.drift = cfg, pab, drift
        self.device = torch.device(device)
        self.stream = stream or torch.cuda.current_stream(self.device)
        ranges = list(cfg.ranges) if pab else [0] * len(cfg.kinds)
        self.recompute, self.source, self.counts = lib.pab_plan_schedule(cfg.N, ranges)
        self.T = len(cfg.kinds)
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        # Cache: two O-sized slots per (block, type), resident in HBM.
        # The cache lives in HBM for the whole trajectory (two slots per
        # block and type; 29.5 GB for the 28-block stack at 480p): check it
        # fits before allocating it.
        if self.device.type == "cuda":
            check_capacity(cache_bytes(cfg), torch.cuda.mem_get_info(self.device)[0],
                           f"broadcast cache of {cfg.name}")
        out_shape = (cfg.B, cfg.F * cfg.S, cfg.C) if cfg.module else cfg.video_shape
        self.slots = [[(torch.empty(out_shape, dtype=tdt, device=self.device),
                        torch.empty(out_shape, dtype=tdt, device=self.device))
                       for _ in range(self.T)] for _ in range(cfg.blocks)]
        # Module intermediates (q, k, v, attention output), shared by every
        # (block, type): the dispatches run one after another on one stream.
        # k and v also hold a cross module's projected text, which can be the
        # larger of the two (more text tokens than video tokens).
        if cfg.module:
            nv, nt = int(np.prod(cfg.video_shape)), int(np.prod(cfg.text_shape))
            self.mod_scratch = [torch.empty(n, dtype=tdt, device=self.device)
                                for n in (nv, max(nv, nt), max(nv, nt), nv)]
        else:
            self.mod_scratch = None
        # Constant text (a module workload with const_text): the text K/V of
        # each block are projected once per trajectory into buffers of their
        # own, and the cross modules read them instead of projecting again.
        self.text_kv = ([(torch.empty(cfg.text_shape, dtype=tdt, device=self.device),
                          torch.empty(cfg.text_shape, dtype=tdt, device=self.device))
                         for _ in range(cfg.blocks)]
                        if cfg.module and cfg.const_text and "cross" in cfg.kinds else None)
        n = int(np.prod(cfg.video_shape))
        self.ws = torch.empty(lib.pab_mse_workspace_bytes(n), dtype=torch.uint8, device=self.device)
        self.drift_out = torch.zeros((cfg.blocks, self.T, cfg.N), dtype=torch.float64,
                                     device=self.device)
        self.inputs = inputs
        # One single-type step descriptor per (block, type), so each type's
        # kernel can be bracketed by events of its own.
        self._rec_cols = [np.ascontiguousarray(self.recompute[:, a]) for a in range(self.T)]
        self._text_len = (np.ascontiguousarray(np.asarray(cfg.text_len, dtype=np.int32))
                          if cfg.text_len is not None else None)
        self._descs = []
        self._types = []
        for b in range(cfg.blocks):
            row = []
            for a in range(self.T):
                t = (lib.TypeDesc * 1)()
                t[0].kind = lib.KINDS[cfg.kinds[a]]
                t[0].slot[0] = self.slots[b][a][0].data_ptr()
                t[0].slot[1] = self.slots[b][a][1].data_ptr()
                t[0].B, t[0].H, t[0].F, t[0].S, t[0].D = cfg.video_shape
                t[0].L = cfg.L if cfg.kinds[a] == "cross" else 0
                t[0].drift = None
                if cfg.kinds[a] == "cross" and cfg.text_len is not None:
                    t[0].text_len = self._text_len.ctypes.data_as(C.POINTER(C.c_int32))
                if cfg.module:
                    for j in range(4):
                        t[0].scratch[j] = self.mod_scratch[j].data_ptr()
                d = lib.StepDesc(
                    num_steps=cfg.N, num_types=1,
                    recompute=self._rec_cols[a].ctypes.data_as(C.POINTER(C.c_uint8)),
                    types=C.cast(t, C.POINTER(lib.TypeDesc)),
                    dtype=lib.PAB_BF16 if cfg.dtype == "bf16" else lib.PAB_F32,
                    softmax_scale=0.0, workspace=self.ws.data_ptr(),
                    workspace_bytes=self.ws.numel(), stream=self.stream.cuda_stream)
                row.append(d)
                self._types.append(t)
            self._descs.append(row)

    def replan(self):
        """Plan the schedule again (as a trajectory does before its first
        step) and check it is the one the descriptors were built on."""
        ranges = list(self.cfg.ranges) if self.pab else [0] * len(self.cfg.kinds)
        rec, _, _ = lib.pab_plan_schedule(self.cfg.N, ranges)
        if not np.array_equal(rec, self.recompute):
            raise RuntimeError("the schedule changed between plans")

    def steps_needed(self):
        return [(b, a, i) for b in range(self.cfg.blocks) for a in range(self.T)
                for i in range(self.cfg.N) if self.recompute[i, a]]

    def cache_state(self):
        """Host copies of every cache slot and of the drift record: with the
        plan, everything a later run needs to continue the trajectory (the
        dispatcher itself keeps no state)."""
        import torch

        torch.cuda.synchronize(self.device)
        return {"slots": [[(s0.cpu(), s1.cpu()) for s0, s1 in row] for row in self.slots],
                "drift": self.drift_out.cpu()}

    def restore_cache(self, state):
        """Load a ``cache_state`` into this trajectory's own slots."""
        for row, saved in zip(self.slots, state["slots"]):
            for (s0, s1), (h0, h1) in zip(row, saved):
                s0.copy_(h0)
                s1.copy_(h1)
        self.drift_out.copy_(state["drift"])

    def run(self, events: bool = False, on_step=None, max_steps=None, first_step=0):
        """Run the trajectory (its first ``max_steps`` steps if given; from
        ``first_step`` on, with the cache slots as the earlier steps left
        them, to resume).
        Returns a dict with the dispatch masks, output pointers and (if
        events) per-type dispatch brackets: brackets["attn"][a] holds one event
        pair per recompute, and brackets["diff"][a] says for each whether it
        also took the attention difference (drift on, a predecessor exists)."""
        import torch

        cfg = self.cfg
        masks = np.zeros((cfg.blocks, cfg.N), dtype=np.uint32)
        outs = [[[None] * self.T for _ in range(cfg.N)] for _ in range(cfg.blocks)]
        brackets = {"attn": [[] for _ in range(self.T)], "diff": [[] for _ in range(self.T)]}
        done = np.zeros((cfg.blocks, self.T), dtype=bool)  # a recompute happened this run
        mk = (lambda: torch.cuda.Event(enable_timing=True)) if events else None
        text_done = set()  # blocks whose constant text K/V this run has projected
        n_run = cfg.N if max_steps is None else min(max_steps, cfg.N)
        # The recomputes in run order: with streamed inputs each one draws
        # the next one's inputs ahead of its own dispatch.
        order = [(b, a, i) for i in range(first_step, n_run) for b in range(cfg.blocks)
                 for a in range(self.T) if self.recompute[i, a]]
        ahead = dict(zip(order, order[1:]))
        # A resumed run: types recomputed before first_step have a predecessor.
        for a in range(self.T):
            if self.recompute[:first_step, a].any():
                done[:, a] = True
        with torch.cuda.stream(self.stream):
            for i in range(first_step, n_run):
                for b in range(cfg.blocks):
                    for a in range(self.T):
                        d = self._descs[b][a]
                        t = self._types[b * self.T + a]
                        rec = bool(self.recompute[i, a])
                        nxt = ahead.get((b, a, i))
                        if rec and cfg.module:
                            x = self.inputs.get(b, a, i, ahead=nxt)
                            w_in, w_kv, w_out = self.inputs.weights(b, a)
                            t[0].x = x[0].data_ptr()
                            t[0].x_text = x[1].data_ptr() if len(x) > 1 else None
                            t[0].w_in, t[0].w_out = w_in.data_ptr(), w_out.data_ptr()
                            t[0].w_kv = w_kv.data_ptr() if w_kv is not None else None
                            if self.text_kv is not None and len(x) > 1:
                                tk, tv = self.text_kv[b]
                                if b not in text_done:
                                    lib.pab_proj_in(x[1], w_kv, [tk, tv], 1, cfg.L, cfg.H, cfg.D,
                                                    stream=self.stream)
                                    text_done.add(b)
                                t[0].x_text = None
                                t[0].scratch[1], t[0].scratch[2] = tk.data_ptr(), tv.data_ptr()
                        elif rec:
                            q, k, v = self.inputs.get(b, a, i, ahead=nxt)
                            t[0].q, t[0].k, t[0].v = q.data_ptr(), k.data_ptr(), v.data_ptr()
                        # With drift on, the dispatcher itself takes the
                        # attention difference of each recompute against the
                        # previous one of its type (into drift_out[b, a, i]).
                        t[0].drift = self.drift_out[b, a].data_ptr() if self.drift else None
                        if events and rec:
                            e0, e1 = mk(), mk()
                            e0.record(self.stream)
                        mask, ptrs = lib.pab_step_dispatch(d, i)
                        if events and rec:
                            e1.record(self.stream)
                            brackets["attn"][a].append((e0, e1))
                            brackets["diff"][a].append(bool(self.drift and done[b, a]))
                        if rec:
                            done[b, a] = True
                        masks[b, i] |= mask << a
                        outs[b][i][a] = ptrs[0]
                if on_step is not None:
                    on_step(i, outs)
        return {"masks": masks, "outs": outs, "brackets": brackets}

    def capture(self):
        """Record the whole trajectory as one HIP graph on this trajectory's
        stream and return it (``torch.cuda.CUDAGraph``) with the dispatch
        record of the captured pass.  ``graph.replay()`` on that stream then
        re-issues every dispatch of the trajectory -- recomputes, attention
        differences, projections -- with one host call; a broadcast step
        records nothing, as it launches nothing.  The dispatch path makes
        no allocation, memset or synchronization, so all of it is captured.
        Capture needs resident inputs (streamed ones are drawn by the host
        loop as it goes) and a stream other than the default one; run the
        trajectory once eagerly first, so that lazily made module weights
        exist before capture."""
        import torch

        if not self.inputs.resident:
            raise ValueError("graph capture needs resident inputs")
        if self.stream.cuda_stream == 0:
            raise ValueError("graph capture needs a stream other than the default stream")
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(graph, stream=self.stream):
            rec = self.run()
        return graph, rec

    def slot_tensor(self, b, a, ptr):
        """The cache slot tensor that lives at device address ``ptr``."""
        for s in self.slots[b][a]:
            if s.data_ptr() == ptr:
                return s
        raise KeyError(ptr)

    def flops(self) -> int:
        """Algorithmic flops this trajectory executes (attention, plus the
        projections of a module configuration)."""
        per = lambda k: attn_flops(self.cfg, k) + (proj_flops(self.cfg, k) if self.cfg.module
                                                    else 0)
        return sum(int(self.counts[a]) * per(k) * self.cfg.blocks
                   for a, k in enumerate(self.cfg.kinds))


# --------------------------------------------------------------- calibration

def calibrate(traj: Trajectory, candidate_ranges=None, rerun: bool = True):
    """Broadcast ranges from a profiling trajectory's attention difference.

    ``traj`` must be a PAB-off trajectory (every step computes) with inputs
    attached.  With ``rerun`` it is run once with the attention-difference
    MSE after every step (the Figure 1 quantity); otherwise the differences
    its last drift-on run left in ``traj.drift_out`` are used.
    ``pab_plan_calibrate`` turns every block's differences into per-type
    ranges (scores averaged over the blocks, which share one schedule), the
    candidates (default: the configuration's ranges) handed out by rank.
    Returns (ranges, scores, diff[blocks, N, T]).
    """
    import torch

    if traj.pab:
        raise ValueError("calibration needs a trajectory that computes every step")
    cfg = traj.cfg
    if rerun:
        keep = traj.drift
        traj.drift = True
        try:
            traj.run(events=False)
        finally:
            traj.drift = keep
    torch.cuda.synchronize(traj.device)
    diff = traj.drift_out.transpose(1, 2).contiguous().cpu().numpy()
    cand = list(cfg.ranges) if candidate_ranges is None else list(candidate_ranges)
    ranges, scores = lib.pab_plan_calibrate(diff, cand)
    return ranges, scores, diff
