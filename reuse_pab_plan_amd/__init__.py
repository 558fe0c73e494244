"""MI355X-native Pyramid Attention Broadcast (PAB) attention hot path.

The compute lives in ``libpab.so`` (hand-written gfx950 HIP kernels behind a
C ABI, declared in ``include/pab.h``).  This package is a thin ctypes binding
(``reuse_pab_plan_amd.lib``), the seeded synthetic-input generator
(``reuse_pab_plan_amd.synth``) and the trajectory harness
(``reuse_pab_plan_amd.harness``).  Importing the package loads nothing; the
library is opened on first use and a missing library is an error, never a
fallback.
"""

__all__ = ["lib", "synth", "harness"]
