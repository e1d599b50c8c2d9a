"""Pins for the oracle's Philox generator (oracle/philox.py).

The pages give no generator; the uniforms follow the Philox-4xW-10 definition of
Salmon et al. (SC'11).  Pins, none of which re-types the oracle's own formula:
  * the Weyl increments re-derived from the golden ratio and sqrt(3);
  * the generic round structure run with 64-bit constants against NumPy's
    Philox (4x64-10), a library implementation of the same family;
  * the 32-bit generator against rocRAND's Philox4x32-10 engine, compiled from
    its header at test time;
  * the uniforms: exact float32 values in [0, 1), chi-square uniform.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle.philox import (PHILOX4x32, PHILOX4x64, philox4x32_10, philox_block,
                           verify_uniforms)


def test_weyl_constants_from_golden_ratio_and_sqrt3():
    for cfg in (PHILOX4x32, PHILOX4x64):
        w = cfg["bits"]
        # floor(2^w * (sqrt(5) - 1) / 2) and floor(2^w * (sqrt(3) - 1)) in integers
        s5 = math.isqrt(5 << (2 * w))
        s3 = math.isqrt(3 << (2 * w))
        assert cfg["weyl"][0] == (s5 - (1 << w)) // 2
        assert cfg["weyl"][1] == s3 - (1 << w)


def test_round_structure_matches_numpy_philox4x64():
    rng = np.random.default_rng(123)
    for _ in range(20):
        ctr = [int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.int64)]
        key = [int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.int64)]
        gen = np.random.Philox(counter=ctr, key=key)
        raw = tuple(int(gen.random_raw()) for _ in range(4))
        # NumPy advances its 256-bit counter before producing the first block
        c = ctr[0] + (ctr[1] << 64) + (ctr[2] << 128) + (ctr[3] << 192) + 1
        words = [(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
        assert philox_block(words, key, **PHILOX4x64) == raw


def test_vectorised_matches_scalar_block():
    rng = np.random.default_rng(7)
    ctr = rng.integers(0, 2**32, size=(64, 4), dtype=np.uint64)
    key = (0xDEADBEEF, 0x01234567)
    got = philox4x32_10(ctr, key)
    for i in range(64):
        assert tuple(int(v) for v in got[i]) == philox_block(ctr[i], key, **PHILOX4x32)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(
    "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"), reason="rocRAND header or g++ missing")
def test_matches_rocrand_philox4x32_10():
    src = r'''
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  unsigned long long seed = strtoull(argv[1], 0, 0), n = strtoull(argv[2], 0, 0),
                     c0 = strtoull(argv[3], 0, 0);
  for (unsigned long long i = 0; i < n; ++i) {
    rocrand_device::philox4x32_10_engine e(seed, 0, 4ull * (c0 + i));
    uint4 r = e.next4();
    printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        cpp, exe = os.path.join(d, "rr.cpp"), os.path.join(d, "rr")
        open(cpp, "w").write(src)
        subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", cpp, "-o", exe], check=True)
        for seed, c0 in ((0, 0), (0x123456789ABCDEF, 2**32 - 3), (2**64 - 1, 12345)):
            n = 256
            out = subprocess.run([exe, str(seed), str(n), str(c0)], check=True,
                                 capture_output=True, text=True).stdout
            want = np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()],
                            dtype=np.uint64)
            c = np.arange(c0, c0 + n, dtype=np.uint64)
            ctr = np.stack([c & np.uint64(0xFFFFFFFF), c >> np.uint64(32),
                            np.zeros_like(c), np.zeros_like(c)], axis=-1)
            got = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
            np.testing.assert_array_equal(got.astype(np.uint64), want)


def test_uniforms_exact_float32_in_unit_interval_and_uniform():
    u, up = verify_uniforms(seed=2024, offset=10**9, positions=np.arange(10**6))
    for x in (u, up):
        assert x.min() >= 0.0 and x.max() < 1.0
        assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
        counts, _ = np.histogram(x, bins=256, range=(0.0, 1.0))
        assert stats.chisquare(counts).pvalue > 1e-4
    # the two words are distinct streams
    assert np.corrcoef(u, up)[0, 1] < 0.01


def test_uniforms_depend_on_offset_plus_position_only():
    a = verify_uniforms(5, 100, np.arange(50))
    b = verify_uniforms(5, 90, np.arange(10, 60))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    c = verify_uniforms(6, 100, np.arange(50))
    assert not np.array_equal(a[0], c[0])
