"""GPU tests of the broadcast cache and step dispatch through the C ABI.

Over whole trajectories: the dispatch mask equals the oracle's schedule at
every step (bit-exact); at every broadcast step the output is the very slot
written at the source step, with bitwise-identical bytes; recomputed outputs
match the oracle (sampled at full size); the drift MSE the dispatcher
computes equals the oracle MSE of the two outputs; PAB off recomputes every
step.  PAB article, Figure 2 caption (broadcast to the next few steps) and
Figure 1 caption (difference between steps measured by the MSE).
"""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from reuse_pab_plan_amd import harness, lib

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()


def _fingerprint(t):
    """Exact content fingerprint of a device tensor (int64 sums of the bits)."""
    bits = t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    x = bits.to(torch.int64).flatten()
    idx = torch.arange(x.numel(), device=x.device, dtype=torch.int64)
    return (int(x.sum()), int((x * (idx % 65521 + 1)).sum()))


def _sample_check(cfg, kind, q, k, v, out, label):
    B, H, F, S, D = cfg.video_shape
    host = lambda t: t.detach().float().cpu().numpy()
    if kind == "spatial":
        sl = (slice(B - 1, B), slice(H - 1, H), slice(F - 1, F))
        rows = np.arange(0, S, max(1, S // 200))
        ref = oracle.spatial_rows(host(q[sl]), host(k[sl]), host(v[sl]), 0, 0, 0, rows)
        got = host(out[B - 1, H - 1, F - 1])[rows]
    elif kind == "temporal":
        pos = np.arange(0, S, max(1, S // 50))
        ref = oracle.temporal_positions(host(q[0, 0][None, None]), host(k[0, 0][None, None]),
                                        host(v[0, 0][None, None]), 0, 0, pos)
        got = host(out[0, 0])[:, pos]
    else:
        nq = F * S
        rows = np.arange(0, nq, max(1, nq // 1000))
        n_text = cfg.text_len[0] if cfg.text_len else None
        hh = min(1, H - 1)  # the second head, where there is one
        ref = oracle.cross_rows(host(q.view(B, H, nq, D)[0, hh][None, None]),
                                host(k[0, hh][None, None]), host(v[0, hh][None, None]), 0, 0, rows,
                                n_text=n_text)
        got = host(out.view(B, H, nq, D)[0, hh])[rows]
        if cfg.text_len:
            # Every other entry, sampled too (its own number of text tokens).
            for b in range(1, B):
                rb = oracle.cross_rows(host(q.view(B, H, nq, D)[b, 0][None, None]),
                                       host(k[b, 0][None, None]), host(v[b, 0][None, None]), 0, 0,
                                       rows, n_text=cfg.text_len[b])
                gb = host(out.view(B, H, nq, D)[b, 0])[rows]
                eb = gb - rb
                mxb = float(np.abs(eb).max())
                rlb = float(np.linalg.norm(eb) / np.linalg.norm(rb))
                print(f"[parity] {label} entry {b}: max_abs={mxb:.2e} rel_l2={rlb:.2e}", flush=True)
                assert mxb <= 2e-2 and rlb <= 5e-3, (label, b, mxb, rlb)
    err = got - ref
    mx, rl = float(np.abs(err).max()), float(np.linalg.norm(err) / np.linalg.norm(ref))
    tol = (2e-2, 5e-3) if cfg.dtype == "bf16" else (1e-5, 1e-5)
    print(f"[parity] {label}: max_abs={mx:.2e} rel_l2={rl:.2e}", flush=True)
    assert mx <= tol[0] and rl <= tol[1], (label, mx, rl)


def _run_checked(cfg, pab=True, blocks_checked=(0,), check_steps=None, resident=True,
                 max_steps=None, print_blocks=None, reuse_check_steps=()):
    """Run a trajectory and check it as it goes.

    Every step: the dispatch mask equals the oracle schedule (all blocks).
    Every recompute of a block in ``print_blocks`` (default: the checked
    blocks) records a bit fingerprint of the slot; every reuse step of such a
    block must hand back the source step's slot with the same fingerprint.
    At ``check_steps`` the recomputed outputs of ``blocks_checked`` are
    compared with the oracle (sampled rows); at ``reuse_check_steps`` the
    reused outputs are compared with the oracle on the source step's inputs
    (drawn again from their generator counters).
    """
    dev = torch.device("cuda:0")
    traj = harness.Trajectory(cfg, pab=pab, device=dev)
    need = traj.steps_needed()
    if max_steps is not None:
        need = [x for x in need if x[2] < max_steps]
    traj.inputs = harness.Inputs(cfg, need if resident else [], device=dev, resident=resident)
    ranges = list(cfg.ranges) if pab else [0] * len(cfg.kinds)
    rec, src, cnt = oracle.schedule(cfg.N, ranges)
    assert np.array_equal(traj.recompute, rec) and np.array_equal(traj.counts, cnt)
    prints = {}
    w0 = -(-15 * cfg.N // 100)
    check_steps = set(check_steps if check_steps is not None else (0, w0, cfg.N - 1))
    print_blocks = tuple(blocks_checked if print_blocks is None else print_blocks)
    reuse_seen = {"n": 0, "oracle": 0}

    def on_step(i, outs):
        torch.cuda.synchronize()
        for b in sorted(set(print_blocks) | set(blocks_checked)):
            for a, kind in enumerate(cfg.kinds):
                ptr = outs[b][i][a]
                slot = traj.slot_tensor(b, a, ptr)
                j = int(src[i, a])
                if j == i:
                    if b in print_blocks:
                        prints[(b, a, i)] = _fingerprint(slot)
                    if b in blocks_checked and i in check_steps:
                        q, k, v = traj.inputs.get(b, a, i)
                        _sample_check(cfg, kind, q, k, v, slot, f"{cfg.name} b{b} {kind} step {i}")
                else:
                    assert ptr == outs[b][j][a], "reuse must hand back the source slot"
                    if b in print_blocks:
                        assert _fingerprint(slot) == prints[(b, a, j)], "reused bytes changed"
                        reuse_seen["n"] += 1
                    if b in blocks_checked and i in reuse_check_steps:
                        q, k, v = traj.inputs.get(b, a, j)
                        _sample_check(cfg, kind, q, k, v, slot,
                                      f"{cfg.name} b{b} {kind} step {i} (reuses {j})")
                        reuse_seen["oracle"] += 1

    res = traj.run(on_step=on_step, max_steps=max_steps)
    n = cfg.N if max_steps is None else max_steps
    for b in range(cfg.blocks):
        for i in range(n):
            for a in range(len(cfg.kinds)):
                assert ((int(res["masks"][b, i]) >> a) & 1) == rec[i, a]
    # every reuse of a fingerprinted block was checked
    n_reuse = sum(1 for i in range(n) for a in range(len(cfg.kinds)) if not rec[i, a])
    assert reuse_seen["n"] == n_reuse * len(print_blocks)
    if reuse_check_steps:
        assert reuse_seen["oracle"] > 0
    return traj, res


def _fingerprints(traj, res_steps):
    """on_step hook recording every block's and type's output fingerprint."""
    cfg = traj.cfg

    def on_step(i, outs):
        torch.cuda.synchronize()
        for b in range(cfg.blocks):
            for a in range(len(cfg.kinds)):
                res_steps[(b, a, i)] = _fingerprint(traj.slot_tensor(b, a, outs[b][i][a]))
    return on_step


@pytest.mark.parametrize("name,cut", [("tiny", 4), ("b480", 6), ("mod_small", 4), ("mod_small", 6)])
def test_resume_from_cache_checkpoint(name, cut):
    # The dispatcher keeps no state: a trajectory stopped after step `cut`,
    # whose cache slots and drift record are copied to the host and loaded
    # into a fresh trajectory, continues bit for bit like one that never
    # stopped -- including broadcast steps right after the cut, whose source
    # step ran before it (PAB article, Figure 2 caption).
    _need_gpu()
    cfg = harness.CONFIGS[name]
    dev = torch.device("cuda:0")
    print(f"[case] resume {name} after step {cut}", flush=True)
    full = harness.Trajectory(cfg, pab=True, device=dev)
    inputs = harness.Inputs(cfg, full.steps_needed(), device=dev)
    full.inputs = inputs
    want = {}
    full.run(on_step=_fingerprints(full, want))
    want_drift = full.drift_out.cpu()
    del full
    first = harness.Trajectory(cfg, pab=True, device=dev)
    first.inputs = inputs
    first.run(max_steps=cut + 1)
    state = first.cache_state()
    del first
    resumed = harness.Trajectory(cfg, pab=True, device=dev)
    resumed.inputs = inputs
    resumed.restore_cache(state)
    # the first resumed step reuses an output computed before the cut
    assert any(not resumed.recompute[cut + 1, a] for a in range(len(cfg.kinds)))
    got = {}
    resumed.run(first_step=cut + 1, on_step=_fingerprints(resumed, got))
    torch.cuda.synchronize()
    assert set(got) == {k for k in want if k[2] > cut}
    for k, v in got.items():
        assert v == want[k], k
    assert torch.equal(resumed.drift_out.cpu(), want_drift)


def test_tiny_trajectory_every_step():
    _need_gpu()
    cfg = harness.CONFIGS["tiny"]
    _run_checked(cfg, check_steps=range(cfg.N), reuse_check_steps=range(cfg.N))


def test_tiny_trajectory_pab_off():
    _need_gpu()
    cfg = harness.CONFIGS["tiny"]
    traj, res = _run_checked(cfg, pab=False, check_steps=(0, 5, 9))
    assert (traj.counts == cfg.N).all()


def test_b480_trajectory():
    _need_gpu()
    _run_checked(harness.CONFIGS["b480"], reuse_check_steps=(6,))


def test_b720_trajectory():
    # 3600-token frames: recomputes checked at the first step, the window's
    # first step and the last step, a broadcast step against its source.
    _need_gpu()
    _run_checked(harness.CONFIGS["b720"], resident=False, reuse_check_steps=(7,))


def test_full3d_trajectory():
    # Window 8..42 (N = 50); step 9 reuses step 8 for both types.
    _need_gpu()
    _run_checked(harness.CONFIGS["full3d"], resident=False, check_steps=(0, 8, 49),
                 reuse_check_steps=(9,))


def test_cfg480_padded_prompts_trajectory():
    # CFG batch with padded prompts (77 and 1 real text tokens of 120) and
    # constant text K/V, through the dispatcher's per-type text lengths.
    _need_gpu()
    _run_checked(harness.CONFIGS["cfg480"])


def test_stack28_trajectory():
    # The whole 30-step trajectory of the 28-block stack: 28 x 3 x 2 cache
    # slots resident in HBM (29.5 GB), inputs drawn per recompute.  The
    # dispatch mask is checked for every (block, step); every block's reused
    # outputs are the source slots with unchanged bytes through the whole
    # window; blocks 0, 13 and 27 are compared with the oracle at the first
    # step, the window's first step (5), a broadcast step (6, which reuses
    # step 5 for all three types) and the last step (29).
    _need_gpu()
    cfg = harness.CONFIGS["stack28"]
    _run_checked(cfg, blocks_checked=(0, 13, 27), check_steps=(0, 5, 29), resident=False,
                 print_blocks=range(cfg.blocks), reuse_check_steps=(6,))


# Shapes of the drift test: each reaches a different way the dispatcher takes
# the difference.  bf16 attention kernels fold it into their output pass
# (spatial with 64- and 32-row query blocks per wave and with three- and
# four-stage rings, temporal with one and two 32-frame blocks, cross with 1, 2
# and 4 32-key blocks, up to D = 128, and padded prompts, one cross launch per
# batch entry with their partials one after another); a separate pass takes
# it for fp32 and for launches with more blocks than the workspace has
# partials.
DRIFT_CASES = [
    # B, H, F, S, D, L, text_len, dtype
    (1, 2, 4, 96, 72, 40, None, "bf16"),
    (2, 3, 5, 333, 128, 77, None, "bf16"),
    (1, 1, 33, 45, 8, 1, None, "bf16"),
    (2, 2, 2, 517, 40, 128, None, "bf16"),
    (1, 2, 64, 7, 64, 64, None, "bf16"),
    (2, 2, 3, 130, 72, 120, (120, 33), "bf16"),
    (1, 2, 3, 70, 24, 20, None, "f32"),
    # Many tiny sequences: the workspace holds fewer partials than spatial
    # (1024) and cross (128) launch blocks, so those two take the separate
    # pass while temporal (16 blocks) still folds it in.
    (1, 16, 64, 4, 8, 16, None, "bf16"),
]


def _high_word_slots(shape, dev, count=2):
    """``count`` bf16 tensors of ``shape`` whose device addresses have bit 31
    of the low 32-bit word set (views into one pool): kernels that move a
    base address into scalar registers must not sign-extend that word."""
    n = int(np.prod(shape))
    nbytes = 2 * n
    align = 1 << 12
    step = (nbytes + align - 1) // align * align
    total = count * step
    assert total < 1 << 31
    pool = torch.empty((1 << 31) + 2 * total + align, dtype=torch.uint8, device=dev)
    base = pool.data_ptr()
    # First offset (4 KiB aligned) from which all views lie where the low
    # word is in [2^31, 2^32).
    low = base & 0xFFFFFFFF
    if low >= 1 << 31 and low + total < 1 << 32:
        off = 0
    elif low < 1 << 31:
        off = (1 << 31) - low
    else:
        off = (1 << 32) - low + (1 << 31)
    off = (off + align - 1) // align * align
    assert off + total <= pool.numel()
    views = []
    for i in range(count):
        o = off + i * step
        t = pool[o:o + nbytes].view(torch.bfloat16).view(shape)
        assert (t.data_ptr() & 0xFFFFFFFF) >= 1 << 31
        views.append(t)
    return pool, views


@pytest.mark.parametrize("case", DRIFT_CASES, ids=lambda c: "x".join(map(str, c[:6])) +
                         ("-padded" if c[6] else "") + "-" + c[7])
def test_drift_matches_oracle_mse(case):
    _drift_case(case)


@pytest.mark.parametrize("case", [(1, 2, 4, 96, 72, 40, None, "bf16"),
                                  (2, 2, 3, 130, 64, 120, (120, 33), "bf16")],
                         ids=["plain", "padded"])
def test_drift_slots_at_high_addresses(case):
    # Regression: cache slots whose addresses have bit 31 of the low word set,
    # for all three types (each kernel reads the previous output through a
    # base address in scalar registers).  A direct load whose base address was
    # assembled from two readfirstlane results (which return int) once
    # sign-extended that word and faulted.
    _drift_case(case, high_slots=True)


def _drift_case(case, high_slots=False):
    # PAB off: consecutive-step attention differences (the Figure 1 analogue),
    # computed on the device by the dispatcher's own two-slot drift path.
    _need_gpu()
    B, H, F, S, D, L, text_len, dt = case
    print(f"[case] drift {case} high_slots={high_slots}", flush=True)
    cfg = harness.Config("drift", dt, B, H, F, S, D, L, 10,
                         ("spatial", "temporal", "cross"), (0, 0, 0), 1, 12, "drift",
                         text_len=text_len)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    rec, _, _ = lib.pab_plan_schedule(cfg.N, [0, 0, 0])
    inputs = harness.Inputs(cfg, [(0, a, i) for a in range(3) for i in range(cfg.N)], device=dev)
    slots = [(torch.empty(cfg.video_shape, dtype=tdt, device=dev),
              torch.empty(cfg.video_shape, dtype=tdt, device=dev)) for _ in range(3)]
    pool = None
    if high_slots:  # every type's two slots
        pool, hs = _high_word_slots(cfg.video_shape, dev, count=6)
        slots = [(hs[2 * a], hs[2 * a + 1]) for a in range(3)]
    drift = torch.full((3, cfg.N), -1.0, dtype=torch.float64, device=dev)
    n = int(np.prod(cfg.video_shape))
    ws = torch.empty(lib.pab_mse_workspace_bytes(n), dtype=torch.uint8, device=dev)
    lens = None if text_len is None else np.ascontiguousarray(np.asarray(text_len, dtype=np.int32))
    types = (lib.TypeDesc * 3)()
    for a, kind in enumerate(cfg.kinds):
        types[a].kind = lib.KINDS[kind]
        types[a].slot[0] = slots[a][0].data_ptr()
        types[a].slot[1] = slots[a][1].data_ptr()
        types[a].B, types[a].H, types[a].F, types[a].S, types[a].D = cfg.video_shape
        types[a].L = cfg.L
        types[a].drift = drift[a].data_ptr()
        if kind == "cross" and lens is not None:
            types[a].text_len = lens.ctypes.data_as(C.POINTER(C.c_int32))
    stream = torch.cuda.current_stream()
    desc = lib.StepDesc(num_steps=cfg.N, num_types=3,
                        recompute=rec.ctypes.data_as(C.POINTER(C.c_uint8)),
                        types=C.cast(types, C.POINTER(lib.TypeDesc)),
                        dtype=lib.PAB_BF16 if dt == "bf16" else lib.PAB_F32,
                        softmax_scale=0.0, workspace=ws.data_ptr(), workspace_bytes=ws.numel(),
                        stream=stream.cuda_stream)
    prev = [None] * 3
    expect = np.full((3, cfg.N), -1.0)
    for i in range(cfg.N):
        for a in range(3):
            q, k, v = inputs.get(0, a, i)
            types[a].q, types[a].k, types[a].v = q.data_ptr(), k.data_ptr(), v.data_ptr()
        mask, outs = lib.pab_step_dispatch(desc, i)
        assert mask == 0b111
        torch.cuda.synchronize()
        for a in range(3):
            cur = [s for s in slots[a] if s.data_ptr() == outs[a]][0]
            host = cur.double().cpu().numpy()
            if prev[a] is not None:
                expect[a, i] = oracle.mse(host, prev[a])
            prev[a] = host
    got = drift.cpu().numpy()
    assert (got[:, 0] == -1.0).all()  # no predecessor: left untouched
    rel = np.abs(got[:, 1:] - expect[:, 1:]) / expect[:, 1:]
    print(f"[parity] drift {case} max rel err {rel.max():.2e}", flush=True)
    assert rel.max() <= 1e-6
    # The synthetic workload's U shape: outer steps differ more than inner ones.
    assert got[:, 1].min() > 10 * got[:, 4:8].max()


def test_range_calibration_matches_oracle():
    # PAB article, "Implementation" and Figure 1 caption: ranges follow each
    # type's consecutive-step attention difference in the stable window.  The
    # PAB-off tiny trajectory runs on the device with the drift MSE after
    # every step; the C planner's calibration of those differences must equal
    # the oracle's calibration of the same numbers bit for bit, and the
    # oracle's own trajectory (fp64 attention and MSE on the exact inputs the
    # device consumed) must give the same ranges.
    _need_gpu()
    cfg = harness.CONFIGS["tiny"]
    dev = torch.device("cuda:0")
    traj = harness.Trajectory(cfg, pab=False, device=dev)
    traj.inputs = harness.Inputs(cfg, traj.steps_needed(), device=dev)
    ranges, scores, diff = harness.calibrate(traj)
    assert diff.shape == (1, cfg.N, len(cfg.kinds))
    want_r, want_s = oracle.calibrate_ranges(diff[0].tolist(), list(cfg.ranges))
    assert list(ranges) == want_r and list(scores) == want_s

    host = lambda t: t.detach().cpu().numpy()

    def inputs_fn(i, a):
        q, k, v = traj.inputs.get(0, a, i)
        return {"q": host(q), "k": host(k), "v": host(v)}

    ref = oracle.trajectory(cfg.N, list(cfg.kinds), [0] * len(cfg.kinds), inputs_fn)
    ref_diff = [[0.0 if d is None else d for d in row] for row in ref["drift"]]
    ref_r, ref_s = oracle.calibrate_ranges(ref_diff, list(cfg.ranges))
    rel = np.abs(np.array(scores) - np.array(ref_s)) / np.array(ref_s)
    print(f"[parity] calibration ranges {list(ranges)} (oracle {ref_r}), "
          f"scores {list(scores)}, max rel err {rel.max():.2e}", flush=True)
    assert rel.max() <= 1e-6
    assert list(ranges) == ref_r
