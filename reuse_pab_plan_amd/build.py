"""Build libpab.so in-tree with hipcc for gfx950.

    python -m reuse_pab_plan_amd.build [--jobs N] [--sanitize]

Every source under ``csrc/`` is compiled to ``_build/`` (at the repository
root) and linked into ``reuse_pab_plan_amd/libpab.so``.  The build always
recompiles: it is also the "does it build" check.  No GPU is needed.

``--sanitize`` builds ``reuse_pab_plan_amd/libpab_san.so`` instead (objects in
``_build/san/``): the host code of every source (argument validation, the
planner, the dispatcher, the launchers) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; device code is built as usual.  Load it with the
ASan runtime preloaded and ``PAB_LIB`` pointing at it, e.g.

    LD_PRELOAD=$(python -m reuse_pab_plan_amd.build --print-asan-runtime) \
    ASAN_OPTIONS=detect_leaks=0 PAB_LIB=reuse_pab_plan_amd/libpab_san.so \
    python -m pytest tests -m "not gpu"
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpab.so")
LIB_SAN = os.path.join(PKG, "libpab_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ASAN_RUNTIME = "/opt/rocm/llvm/lib/clang/{v}/lib/linux/libclang_rt.asan-x86_64.so"
# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]

SOURCES = [
    "abi.cpp",
    "plan.cpp",
    "dispatch.cpp",
    "mse.hip",
    "attn_f32.hip",
    "spatial.hip",
    "cross.hip",
    "temporal.hip",
    "proj.hip",
    "peaks.hip",
    "synth.hip",
]

# Packed fp32 instructions are disabled for all device code on purpose.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS addresses are 32-bit on the device; the host pass (64-bit pointers)
    # would warn on every cast of one to an LDS pointer it never compiles.
    "-Xarch_host", "-Wno-int-to-pointer-cast",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The spatial kernel's row maxima see no NaN (scores
# of finite inputs, masked entries are -inf), so its max needs no NaN
# quieting: this drops a canonicalizing VALU op per max chain.  (Its finite
# tests read exponent bits, which this flag leaves alone.)
EXTRA = {
    "spatial.hip": ["-fno-honor-nans"],
}


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime of the ROCm toolchain."""
    base = "/opt/rocm/llvm/lib/clang"
    versions = sorted(os.listdir(base)) if os.path.isdir(base) else []
    for v in reversed(versions):
        path = ASAN_RUNTIME.format(v=v)
        if os.path.exists(path):
            return path
    raise RuntimeError("no libclang_rt.asan-x86_64.so under " + base)


def _compile(src: str, sanitize: bool = False) -> tuple[str, float, str]:
    t0 = time.time()
    out_dir = os.path.join(BUILD, "san") if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(SAN_FLAGS if sanitize else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in line  # host pass does not know the device feature
    )
    if "warning:" not in out and "error" not in out:
        out = ""
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{out}")
    return obj, time.time() - t0, out


def build(jobs: int | None = None, verbose: bool = True, sanitize: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "san") if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    for (obj, dt, out), src in zip(results, SOURCES):
        if verbose:
            print(f"[build] {src:16s} {dt:6.1f}s", flush=True)
        if out.strip() and verbose:
            print(out, flush=True)
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(SAN_FLAGS if sanitize else []), "-o",
           tmp, *[r[0] for r in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"[build] wrote {lib}", flush=True)
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--sanitize", action="store_true",
                    help="build libpab_san.so with host-side ASan/UBSan")
    ap.add_argument("--print-asan-runtime", action="store_true",
                    help="print the ASan runtime to preload and exit")
    args = ap.parse_args(argv)
    if args.print_asan_runtime:
        print(asan_runtime())
        return 0
    build(args.jobs, sanitize=args.sanitize)
    return 0


if __name__ == "__main__":
    sys.exit(main())
