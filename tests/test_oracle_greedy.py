"""Pins for the oracle's greedy acceptance.

The pages fix one property exactly: greedy speculative decoding gives the
same output as greedy decoding with the target alone ("Inference-4",
Draft-model speculative decoding, greedy bullet and the listing's
docstring).  A tiny context-dependent toy target makes that checkable by
brute force: for a few prefixes, every one of the V^K draft sequences goes
through the verify step, and each output must be the next n+1 tokens of
target-only greedy decoding, with n the length of the longest draft prefix
that greedy decoding would also have produced.
"""
import itertools
import zlib

import numpy as np
import pytest

from oracle.verify import accept_greedy

V, K, H = 8, 3, 16


class ToyTarget:
    """logits(prefix) = W · h(prefix), h a seeded hash of the token prefix."""

    def __init__(self, seed):
        self.W = np.random.default_rng(seed).normal(size=(V, H))

    def logits(self, prefix):
        key = zlib.crc32(np.asarray(prefix, np.int64).tobytes())
        h = np.random.default_rng(key).normal(size=H)
        return self.W @ h

    def greedy(self, prefix, n):
        seq = list(prefix)
        for _ in range(n):
            seq.append(int(np.argmax(self.logits(seq))))
        return seq[len(prefix):]


@pytest.mark.parametrize("seed,prefix", [(0, [1, 2, 3]), (1, [5]), (2, [0, 0, 7, 4]), (3, [6, 1])])
def test_bruteforce_equals_target_only_greedy(seed, prefix):
    tgt = ToyTarget(seed)
    ref = tgt.greedy(prefix, K + 1)
    drafts = np.array(list(itertools.product(range(V), repeat=K)), np.int64)   # [V^K, K]
    B = len(drafts)
    logits = np.empty((B, K + 1, V))
    for b, d in enumerate(drafts):
        for i in range(K + 1):
            logits[b, i] = tgt.logits(list(prefix) + list(d[:i]))
    res = accept_greedy(logits, drafts)
    for b, d in enumerate(drafts):
        n = 0
        while n < K and d[n] == ref[n]:
            n += 1
        assert res.accepted_len[b] == n
        assert list(res.out_tokens[b, :n + 1]) == ref[:n + 1]
        assert np.all(res.out_tokens[b, n + 1:] == -1)
    # at least one draft sequence accepts everything and earns the bonus token
    assert np.sum(res.accepted_len == K) == 1


def test_ties_take_lowest_index():
    z = np.array([[[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]]])
    res = accept_greedy(z, np.array([[1]]))
    assert res.argmax[0].tolist() == [1, 0]
    assert res.accepted_len[0] == 1 and res.out_tokens[0].tolist() == [1, 0]
    assert res.margin[0].tolist() == [0.0, 0.0]


def test_k0_is_plain_argmax():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(4, 1, 50))
    res = accept_greedy(z, np.zeros((4, 0), np.int64))
    assert np.all(res.accepted_len == 0)
    np.testing.assert_array_equal(res.out_tokens[:, 0], np.argmax(z[:, 0], -1))


def test_margin_is_top1_minus_top2():
    rng = np.random.default_rng(4)
    z = rng.normal(size=(3, 4, 20))
    res = accept_greedy(z, rng.integers(0, 20, size=(3, 3)))
    s = np.sort(z, axis=-1)
    np.testing.assert_allclose(res.margin, s[..., -1] - s[..., -2], rtol=0, atol=0)


def test_bad_rows_and_row_subset():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(5, 3, 10))
    d = np.argmax(z[:, :2], -1)
    d[1, 0] = 10                       # out of range
    z[2, 2, 3] = np.nan                # NaN anywhere in the row
    z[3, 1, :] = -np.inf               # a position with no finite logit
    res = accept_greedy(z, d, rows=[0, 1, 2, 3])
    assert res.accepted_len.tolist() == [2, -1, -1, -1, -2]
    assert np.all(res.out_tokens[1:] == -1)
    assert res.out_tokens[0].tolist() == list(d[0]) + [int(np.argmax(z[0, 2]))]
