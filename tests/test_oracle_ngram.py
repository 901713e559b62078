"""Pins of the oracle's prompt-lookup drafter.

  * hand-worked sequences whose drafts follow from the rule by inspection;
  * an independent formulation: the token sequence is written as text (one
    fixed-width field per token) and Python's str.rfind finds the most recent
    earlier occurrence of each suffix n-gram, longest first;
  * invariants on random copy-heavy sequences: the proposed tokens follow an
    occurrence of the matched suffix, no later occurrence of it exists, and
    no longer suffix occurs earlier.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("seq,k,g,drafts,n", [
    ([1, 2, 3, 4, 1, 2, 3], 3, 3, [4, 1, 2], 3),        # trigram 1 2 3 seen at 0 -> 4 1 2
    ([1, 2, 3, 4, 1, 2, 3], 9, 3, [4, 1, 2, 3], 3),     # fewer drafts when the sequence ends
    ([5, 9, 5, 7, 9, 5], 2, 3, [7, 9], 2),              # 7 9 5 not seen; 9 5 at 1 -> 7 9
    ([5, 9, 5, 7, 8, 5], 2, 3, [7, 8], 1),              # only the unigram 5, most recent at 2
    ([4, 4, 4, 4], 5, 2, [4], 2),                       # bigram 4 4: most recent window j = 1
    ([1, 2, 3], 4, 3, [], 0),                           # nothing repeats
    ([7], 4, 3, [], 0),                                 # L = 1: nothing before the last token
    ([], 4, 3, [], 0),
    ([3, 1, 3], 2, 1, [1, 3], 1),                       # unigram 3 at 0 -> 1 3
])
def test_worked_sequences(seq, k, g, drafts, n):
    d, m = oracle.ngram_propose_one(seq, k, g)
    assert d.tolist() == drafts and m == n


def _by_rfind(seq, k, g):
    text = "".join("%08x," % (t & 0xFFFFFFFF) for t in seq)
    w = 9
    L = len(seq)
    for n in range(g, 0, -1):
        if L <= n:
            continue
        suffix = text[(L - n) * w:]
        # occurrences must start before position L-n and end before the last token
        pos = text.rfind(suffix, 0, (L - 1) * w)
        while pos >= 0 and pos % w:
            pos = text.rfind(suffix, 0, pos + len(suffix) - 1)
        if pos >= 0:
            start = pos // w + n
            return list(seq[start:start + k]), n
    return [], 0


def _copy_heavy(rng, L, V):
    s = list(rng.integers(0, V, min(L, 50)))
    while len(s) < L:
        if rng.random() < 0.6 and len(s) > 10:
            a = int(rng.integers(0, len(s) - 5))
            s.extend(s[a:a + int(rng.integers(3, 30))])
        else:
            s.extend(rng.integers(0, V, int(rng.integers(1, 20))).tolist())
    return np.array(s[:L], np.int64)


@pytest.mark.parametrize("seed", range(6))
def test_matches_independent_string_search(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        L = int(rng.integers(0, 400))
        V = int(rng.choice([3, 20, 50000]))
        s = _copy_heavy(rng, L, V)
        k, g = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        d, n = oracle.ngram_propose_one(s, k, g)
        rd, rn = _by_rfind(s.tolist(), k, g)
        assert (d.tolist(), n) == (rd, rn), (s.tolist(), k, g)


def test_invariants_and_batch_form():
    rng = np.random.default_rng(11)
    hist = [_copy_heavy(rng, int(rng.integers(0, 3000)), 1000) for _ in range(30)]
    drafts, count, matched, row_start = oracle.ngram_propose(hist, 7, 4)
    assert row_start[0] == 0 and np.all(np.diff(row_start) == count + 1)
    for b, s in enumerate(hist):
        n, c = int(matched[b]), int(count[b])
        assert np.all(drafts[b, c:] == -1)
        if n == 0:
            assert c == 0
            continue
        L = len(s)
        suf = s[L - n:]
        occ = [j for j in range(0, L - n) if np.array_equal(s[j:j + n], suf)]
        start = occ[-1] + n
        assert drafts[b, :c].tolist() == s[start:start + c].tolist() and c == min(7, L - start)
        for m in range(n + 1, 5):      # no longer suffix occurs earlier
            if L > m:
                assert not any(np.array_equal(s[j:j + m], s[L - m:]) for j in range(0, L - m))


@pytest.mark.parametrize("seed", range(4))
def test_trailing_runs_brute_force(seed):
    """run(e) against a direct count of agreeing tokens, walking back from e
    and from the sequence's end one token at a time."""
    rng = np.random.default_rng(100 + seed)
    for _ in range(60):
        L = int(rng.integers(0, 40))
        s = rng.integers(0, int(rng.choice([2, 3, 6])), L)
        g = int(rng.integers(1, 7))
        want = []
        for e in range(L - 1):
            k = 0
            while k < g and e - k >= 0 and s[e - k] == s[L - 1 - k]:
                k += 1
            want.append(k)
        assert oracle.trailing_runs(s, g).tolist() == want, (s.tolist(), g)
