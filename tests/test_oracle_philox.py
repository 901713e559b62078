"""Pins for the oracle's Philox4x32-10 and its uniforms.

1. Published known-answer blocks of Philox4x32-10 (the known-answer test
   vectors distributed with the Random123 library that accompanies Salmon et
   al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).
2. rocRAND's own Philox4x32-10 engine (an independent implementation, run as
   host code on the CPU) on thousands of random (counter, key) pairs.
3. The 24-bit uniform grid: exact values, range, and a Kolmogorov-Smirnov
   test of uniformity over 10^6 draws.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x32_10, uniform24, verify_uniforms

# (counter c0..c3, key k0 k1) -> output block, Philox4x32 with 10 rounds.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_known_answer_blocks(ctr, key, expect):
    out = philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
    assert tuple(int(x) for x in out) == expect


def _rocrand_blocks(tmp_path, ctrs, keys):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    src = os.path.join(os.path.dirname(__file__), "philox_rocrand_blocks.cpp")
    exe = str(tmp_path / "philox_rocrand_blocks")
    # host-only build: -x hip for the HIP vector types, but nothing is launched
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", src, "-o", exe],
                   check=True, capture_output=True)
    lines = "\n".join("%x %x %x %x %x %x" % (*c, *k) for c, k in zip(ctrs, keys))
    res = subprocess.run([exe], input=lines, capture_output=True, text=True, check=True)
    return np.array([[int(w, 16) for w in ln.split()] for ln in res.stdout.strip().splitlines()],
                    dtype=np.uint64).astype(np.uint32)


def test_against_rocrand_engine(tmp_path):
    rng = np.random.default_rng(12345)
    n = 4000
    ctrs = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    keys = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    # also the small counters the verify step actually uses
    ctrs[:64] = np.stack([np.arange(64), np.arange(64) % 7, np.zeros(64), np.zeros(64)], -1)
    ref = _rocrand_blocks(tmp_path, ctrs, keys)
    got = philox4x32_10(ctrs, keys)
    assert ref.shape == got.shape
    np.testing.assert_array_equal(got, ref)


def test_uniform24_grid():
    w = np.array([0, 255, 256, 0xFFFFFFFF, 0x80000000], np.uint32)
    u = uniform24(w)
    assert u[0] == 0.0 and u[1] == 0.0
    assert u[2] == 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24          # largest value, strictly below 1
    assert u[4] == 0.5
    # every value is a multiple of 2^-24 and exact in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_verify_uniforms_uniform_ks():
    seeds = np.arange(250_000, dtype=np.uint64)
    u, u2 = verify_uniforms(seeds[:, None], np.uint64(3), np.arange(4)[None, :])
    for arr in (u.ravel(), u2.ravel()):
        assert arr.min() >= 0.0 and arr.max() < 1.0
        assert stats.kstest(arr, "uniform").pvalue > 1e-3
    # the accept and terminal words are uncorrelated
    assert abs(np.corrcoef(u.ravel(), u2.ravel())[0, 1]) < 0.01


def test_verify_uniforms_layout():
    """Counter = (pos, seq, 0, 0), key = (seed lo, seed hi): a different
    position, sequence or either half of the seed gives a different block."""
    seed = np.uint64(0x0123456789ABCDEF)
    base = verify_uniforms(seed, 5, 2)
    for s, b, i in [(seed, 5, 3), (seed, 6, 2), (seed ^ np.uint64(1), 5, 2),
                    (seed ^ np.uint64(1 << 40), 5, 2)]:
        assert verify_uniforms(s, b, i)[0] != base[0]
    blk = philox4x32_10(np.array([2, 5, 0, 0], np.uint32), np.array([0x89ABCDEF, 0x01234567], np.uint32))
    assert base[0] == (int(blk[0]) >> 8) * 2.0 ** -24
    assert base[1] == (int(blk[1]) >> 8) * 2.0 ** -24
