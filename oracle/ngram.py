"""fp-free CPU definition of the prompt-lookup (n-gram) drafter.

Prompt lookup decoding drafts without a model: take the last n tokens of the
sequence, look for the same n tokens earlier in the sequence (prompt and
generated text alike), and propose the tokens that followed the most recent
earlier occurrence; longer n-grams are preferred, and a sequence whose
n-grams never occurred before gets no drafts ("Inference-4", Prompt lookup
decoding, text; "What is speculative decoding" guide, the n-gram simple
method).

Written from that rule.  An earlier occurrence of an n-gram is a window of n
tokens that ends before the last token of the sequence s (length L), i.e. at
an end position e <= L-2.  For each such e let run(e) be how many tokens,
walking backwards from e and from the end of the sequence in step, agree:
s[e-k] == s[L-1-k] for k = 0 .. run(e)-1, counted up to max_ngram.  The
window of n tokens ending at e repeats the final n-gram exactly when
run(e) >= n.  So the longest final n-gram that occurred earlier has length
n* = max_e run(e), and its most recent occurrence ends at the largest e with
run(e) = n*; the drafts are the tokens after it, s[e+1 .. e+n_drafts], fewer
when the sequence ends first.  n* = 0 (no end position shares even the last
token) means no drafts.  Only token equality is involved: no rounding.

Part of the oracle (test infrastructure); see oracle/__init__.py.
"""
from __future__ import annotations

import numpy as np


def trailing_runs(seq, max_ngram: int) -> np.ndarray:
    """run(e) for every end position e = 0 .. L-2 of one sequence: the number
    of consecutive tokens, backwards from e and from the sequence's end in
    step, that agree, at most max_ngram."""
    s = np.asarray(seq, dtype=np.int64).reshape(-1)
    L = len(s)
    ends = np.arange(max(L - 1, 0))
    run = np.zeros(len(ends), np.int64)
    alive = np.ones(len(ends), bool)          # every earlier offset agreed
    for k in range(min(max_ngram, max(L - 1, 0))):
        inside = ends >= k                    # s[e-k] exists
        back = s[np.where(inside, ends - k, 0)]
        alive &= inside & (back == s[L - 1 - k])
        run += alive
    return run


def ngram_propose_one(seq, n_drafts: int, max_ngram: int):
    """Drafts (int64 array, possibly empty) and the n-gram length that
    matched (0 if none) for one sequence."""
    s = np.asarray(seq, dtype=np.int64).reshape(-1)
    run = trailing_runs(s, max_ngram)
    best = int(run.max()) if len(run) else 0
    if best == 0:
        return s[:0].copy(), 0
    e = int(np.max(np.flatnonzero(run == best)))     # most recent end position of the longest match
    return s[e + 1:e + 1 + n_drafts].copy(), best


def ngram_propose(histories, n_drafts: int, max_ngram: int):
    """Batch form: histories is a list of 1-D token arrays.  Returns
    (drafts [B, n_drafts] int32 padded with -1, draft_count [B] int32,
    matched n [B] int32, row_start [B+1] int32 with row_start[b+1] =
    row_start[b] + draft_count[b] + 1, the packing of the verify rows)."""
    B = len(histories)
    drafts = np.full((B, n_drafts), -1, np.int32)
    count = np.zeros(B, np.int32)
    matched = np.zeros(B, np.int32)
    for b, h in enumerate(histories):
        d, n = ngram_propose_one(h, n_drafts, max_ngram)
        drafts[b, :len(d)] = d
        count[b] = len(d)
        matched[b] = n
    row_start = np.concatenate([[0], np.cumsum(count.astype(np.int64) + 1)]).astype(np.int32)
    return drafts, count, matched, row_start
