"""CPU tests of the seeded workload generator's definition (no GPU).

The device generator (include/pab_synth.h) is Philox4x32-10 (Salmon et al.,
SC'11) followed by the Box-Muller transform; ``synth.philox4x32_10`` and
``synth.philox_normals`` restate it on the host.  Pinned here: the published
known-answer vectors, the counter/key layout of a stream, the uniform
mapping's bounds, and the distribution of the normals (moments, a
Kolmogorov-Smirnov test, independence of the cos/sin pair).  The device
kernels are checked against these host functions in tests/test_gpu_synth.py.
"""

import ctypes as C
import os

import numpy as np
import pytest
from scipy import stats

from reuse_pab_plan_amd import lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kat():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "philox_kat.txt")):
        line = line.split("#")[0].split()
        if line:
            v = [int(x, 16) for x in line]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_philox_known_answer_vectors():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, want in rows:
        got = synth.philox4x32_10(np.array(ctr, dtype=np.uint32), np.array(key, dtype=np.uint32))
        assert [int(x) for x in got] == want, (ctr, key)


def test_philox_rounds_matter():
    # Nine rounds would give a different answer: the vector pins ten rounds,
    # and one flipped counter bit changes about half the output bits.
    base = synth.philox4x32_10(np.zeros(4, dtype=np.uint32), np.zeros(2, dtype=np.uint32))
    flipped = synth.philox4x32_10(np.array([1, 0, 0, 0], dtype=np.uint32),
                                  np.zeros(2, dtype=np.uint32))
    bits = sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(base, flipped))
    assert 40 <= bits <= 88


def test_stream_block_layout():
    # Block i of a stream has counter (lo32(i), hi32(i), 0, 0) and the key's
    # two halves; blocks past 2^32 use the high counter word.
    key = 0x123456789ABCDEF
    for i in (0, 1, 7, 2**32 - 1, 2**32, 2**40 + 3):
        got = synth.philox_blocks(key, i, 1)[0]
        want = synth.philox4x32_10(np.array([i & 0xFFFFFFFF, i >> 32, 0, 0], dtype=np.uint32),
                                   np.array([key & 0xFFFFFFFF, key >> 32], dtype=np.uint32))
        assert np.array_equal(got, want)
    # consecutive blocks, in one call or one by one
    many = synth.philox_blocks(key, 5, 4)
    for j in range(4):
        assert np.array_equal(many[j], synth.philox_blocks(key, 5 + j, 1)[0])


def test_normals_uniform_mapping_bounds():
    # u = ((x >> 9) + 1/2) 2^-23 lies in [2^-24, 1 - 2^-24]: log never sees 0
    # and |z| <= sqrt(2 ln 2^24).
    x = np.array([0, 511, 512, 2**32 - 1], dtype=np.float64)
    u = (np.floor(x / 512) + 0.5) * 2.0 ** -23
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[3] == 1 - 2.0 ** -24
    z = synth.philox_normals(7, 1 << 16)
    assert np.isfinite(z).all() and np.abs(z).max() <= np.sqrt(2 * 24 * np.log(2)) + 1e-12


def test_normals_first_block_by_hand():
    # Element layout: words (0, 1) give elements 0 (cos) and 1 (sin), words
    # (2, 3) give elements 2 and 3.
    key = 99
    w = synth.philox_blocks(key, 0, 1)[0].astype(np.float64)
    u = lambda x: (np.floor(x / 512) + 0.5) * 2.0 ** -23
    r0, r1 = np.sqrt(-2 * np.log(u(w[0]))), np.sqrt(-2 * np.log(u(w[2])))
    want = [r0 * np.cos(2 * np.pi * u(w[1])), r0 * np.sin(2 * np.pi * u(w[1])),
            r1 * np.cos(2 * np.pi * u(w[3])), r1 * np.sin(2 * np.pi * u(w[3]))]
    assert np.allclose(synth.philox_normals(key, 4), want, rtol=0, atol=1e-15)


def test_normals_distribution():
    n = 1 << 20
    z = synth.philox_normals(synth.stream_id(2, 0, 0, 0, -1), n)
    se = 1 / np.sqrt(n)
    assert abs(z.mean()) < 5 * se
    assert abs(z.var() - 1) < 5 * np.sqrt(2) * se
    assert abs(np.mean(z ** 4) - 3) < 5 * np.sqrt(96) * se
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # the cos and sin members of a pair are uncorrelated, and so are
    # neighbouring blocks
    zc, zs = z[0::2], z[1::2]
    assert abs(np.corrcoef(zc, zs)[0, 1]) < 5 / np.sqrt(n // 2)
    assert abs(np.corrcoef(z[:-4], z[4:])[0, 1]) < 5 / np.sqrt(n)


def test_streams_differ():
    a = synth.philox_normals(synth.stream_id(4, 13, 1, 2, 7), 4096)
    b = synth.philox_normals(synth.stream_id(4, 13, 1, 2, 8), 4096)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1


@pytest.mark.skipif(not os.path.exists(lib.LIB_PATH), reason="libpab.so not built")
def test_synth_validation_codes():
    L = lib.load()
    ok = C.c_void_p(0x10000)
    assert L.pab_synth_philox(None, 4, 1, 0, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_philox(C.c_void_p(0x10004), 4, 1, 0, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_philox(ok, 0, 1, 0, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_philox(ok, 4, 1, 2**62 - 2, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(None, 8, lib.PAB_BF16, 1, 1.0, 0, 0.0, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(C.c_void_p(0x10002), 8, lib.PAB_BF16, 1, 1.0, 0, 0.0, None) == \
        lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(ok, 0, lib.PAB_BF16, 1, 1.0, 0, 0.0, None) == lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(ok, 8, lib.PAB_BF16, 1, float("nan"), 0, 0.0, None) == \
        lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(ok, 8, lib.PAB_BF16, 1, 1.0, 2, float("inf"), None) == \
        lib.PAB_ERR_INVALID_ARG
    assert L.pab_synth_normal(ok, 8, 7, 1, 1.0, 0, 0.0, None) == lib.PAB_ERR_UNSUPPORTED
    assert "dtype" in lib.pab_last_error()
