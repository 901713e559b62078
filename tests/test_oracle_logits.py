"""Pins for the oracle's LM-head logits and bf16 widening.

* bf16 bit patterns widen to the IEEE values they encode (closed forms).
* Logits equal exact rational arithmetic (fractions.Fraction) on small
  random slices, to within the fp64 summation bound; on small-integer inputs
  they are exact.  Asymmetric shapes catch a transposed operand.
"""
from fractions import Fraction

import numpy as np

from oracle.verify import lm_head_logits, widen_bf16


def test_widen_bf16_closed_forms():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000, 0x4049], np.uint16)
    v = widen_bf16(bits)
    assert v[0] == 1.0
    assert v[1] == -2.0
    assert v[2] == 1.0 + 2.0 ** -7
    assert v[3] == np.inf and v[4] == -np.inf
    assert v[5] == 2.0 ** -133                 # smallest bf16 subnormal
    assert v[6] == 0.0 and np.signbit(v[7])
    assert v[8] == 3.140625
    nan = widen_bf16(np.array([0x7FC0], np.uint16))
    assert np.isnan(nan[0])


def _bf16_exact(rng, shape, scale):
    """Random values that are exactly representable in bf16."""
    x = (rng.normal(size=shape) * scale).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    return widen_bf16(bits)


def test_logits_match_exact_rationals():
    rng = np.random.default_rng(7)
    M, H, V = 3, 40, 7
    x = _bf16_exact(rng, (M, H), 1.0)
    W = _bf16_exact(rng, (V, H), 0.05)
    got = lm_head_logits(x, W, chunk=3)          # chunk smaller than V: exercises the loop
    assert got.shape == (M, V)
    for m in range(M):
        for v in range(V):
            exact = sum(Fraction(float(x[m, h])) * Fraction(float(W[v, h])) for h in range(H))
            mag = sum(abs(float(x[m, h]) * float(W[v, h])) for h in range(H))
            bound = H * 2.0 ** -53 * mag
            assert abs(Fraction(float(got[m, v])) - exact) <= Fraction(bound)


def test_logits_small_integers_exact():
    rng = np.random.default_rng(8)
    M, H, V = 5, 4096, 33
    x = rng.integers(-4, 5, size=(M, H)).astype(np.float64)
    W = rng.integers(-4, 5, size=(V, H)).astype(np.float64)
    got = lm_head_logits(x, W, chunk=8)
    ref = np.array([[int(np.dot(x[m].astype(np.int64), W[v].astype(np.int64))) for v in range(V)]
                    for m in range(M)], dtype=np.float64)
    np.testing.assert_array_equal(got, ref)


def test_logits_orientation():
    """hidden[m] · W[v] lands at logits[m, v] (one-hot rows make it visible)."""
    M, H, V = 2, 3, 4
    x = np.zeros((M, H))
    x[0, 1] = 1.0
    x[1, 2] = 2.0
    W = np.arange(V * H, dtype=np.float64).reshape(V, H)
    got = lm_head_logits(x, W)
    np.testing.assert_array_equal(got[0], W[:, 1])
    np.testing.assert_array_equal(got[1], 2.0 * W[:, 2])
