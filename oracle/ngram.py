"""fp-free CPU definition of the prompt-lookup (n-gram) drafter.

Prompt lookup decoding drafts without a model: take the last n tokens of the
sequence, look for the same n tokens earlier in the sequence (prompt and
generated text alike), and propose the tokens that followed the most recent
earlier occurrence; longer n-grams are tried first, and a sequence whose
n-grams never occurred before gets no drafts ("Inference-4", Prompt lookup
decoding; "What is speculative decoding" guide, the n-gram simple method).

For a sequence s of length L and n = max_ngram, ..., 1 (skipping n >= L):
the candidate windows are s[j : j+n] for 0 <= j <= L-1-n (every n-gram that
ends before the last token); if any equals s[L-n : L], take the largest such
j, start = j + n, and propose s[start : start + n_drafts] (fewer when the
sequence ends first).  Only token equality is involved: no rounding.

Part of the oracle (test infrastructure); see oracle/__init__.py.
"""
from __future__ import annotations

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view


def ngram_propose_one(seq, n_drafts: int, max_ngram: int):
    """Drafts (int64 array, possibly empty) and the n-gram length that
    matched (0 if none) for one sequence."""
    s = np.asarray(seq, dtype=np.int64).reshape(-1)
    L = len(s)
    for n in range(max_ngram, 0, -1):
        if L <= n:
            continue
        windows = sliding_window_view(s[:-1], n)          # s[j:j+n], j = 0 .. L-1-n
        hits = np.nonzero(np.all(windows == s[L - n:], axis=1))[0]
        if len(hits):
            start = int(hits[-1]) + n
            return s[start:start + n_drafts].copy(), n
    return s[:0].copy(), 0


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
