"""Pins of the oracle's packed-batch rules (per-sequence draft counts K_b).

Each sequence of a packed batch is verified as a dense sequence with K = K_b
in batch slot b.  The pins check that reading against what the dense rule,
already pinned on its own, gives when the batch is built independently:

  * every K_b equal to K: the packed result equals the dense one field by
    field, for both rules and for row subsets;
  * mixed K_b: each sequence equals row b of a dense batch of B sequences with
    K = K_b whose row b holds that sequence's data (so a wrong row offset or
    batch slot shows up);
  * K_b = 0: greedy emits the argmax of the single row; sampled draws the
    inverse CDF of q_0 at the Philox terminal uniform of (seed_b, b, 0),
    computed here from the softmax and a cumulative sum;
  * malformed offsets mark exactly the sequences they name.
"""
import numpy as np
import pytest

import oracle
import synth


def _batch(B, K_max, V, seed, counts=None):
    rng = np.random.default_rng(seed)
    counts = synth.draft_counts(B, K_max, seed) if counts is None else np.asarray(counts, np.int32)
    z = rng.normal(0, 2, (B, K_max + 1, V))
    zd = z[:, :K_max] + rng.normal(0, 1, (B, K_max, V))
    d = rng.integers(0, V, (B, K_max))
    # greedy drafts that often match: copy the target argmax with prob 0.7
    am = np.argmax(z[:, :K_max], axis=-1)
    d = np.where(rng.random((B, K_max)) < 0.7, am, d)
    seeds = rng.integers(0, 2 ** 63, B).astype(np.uint64)
    return counts, z, zd, d, seeds


def _packed(counts, z, zd, d):
    rs = synth.row_start(counts)
    return rs, synth.pack_rows(z, counts), synth.pack_rows(zd, counts, True), synth.pack_rows(d, counts, True)


@pytest.mark.parametrize("K", [0, 1, 5])
def test_uniform_counts_equal_dense(K):
    B, V = 6, 300
    counts, z, zd, d, seeds = _batch(B, K, V, 11 + K, counts=[K] * 6)
    rs, zp, zdp, dp = _packed(counts, z, zd, d)
    for rows in (None, np.array([4, 1, 3])):
        g = oracle.accept_greedy(z, d, rows)
        gr = oracle.accept_greedy_ragged(zp, dp, rs, K, rows)
        np.testing.assert_array_equal(g.accepted_len, gr.accepted_len)
        np.testing.assert_array_equal(g.out_tokens.reshape(-1), gr.out_tokens)
        np.testing.assert_array_equal(g.argmax.reshape(-1), gr.argmax)
        s = oracle.accept_sample(z, zd, d, 0.9, seeds, rows)
        sr = oracle.accept_sample_ragged(zp, zdp, dp, rs, K, 0.9, seeds, rows)
        np.testing.assert_array_equal(s.accepted_len, sr.accepted_len)
        np.testing.assert_array_equal(s.out_tokens.reshape(-1), sr.out_tokens)
        np.testing.assert_array_equal(s.probs_at_draft.reshape(-1, 2), sr.probs_at_draft)
        np.testing.assert_array_equal(s.u_terminal.reshape(-1), sr.u_terminal)
        np.testing.assert_array_equal(s.terminal_margin, sr.terminal_margin)


def test_each_sequence_equals_dense_batch_at_its_slot():
    B, K_max, V, T = 7, 6, 257, 0.8
    counts, z, zd, d, seeds = _batch(B, K_max, V, 5, counts=[3, 0, 6, 1, 0, 5, 2])
    rs, zp, zdp, dp = _packed(counts, z, zd, d)
    gr = oracle.accept_greedy_ragged(zp, dp, rs, K_max)
    sr = oracle.accept_sample_ragged(zp, zdp, dp, rs, K_max, T, seeds)
    rng = np.random.default_rng(99)
    for b in range(B):
        kb = int(counts[b])
        # a dense batch of B sequences with K = kb: unrelated data except row b
        zz = rng.normal(0, 2, (B, kb + 1, V))
        zzd = rng.normal(0, 2, (B, kb, V))
        dd = rng.integers(0, V, (B, kb))
        zz[b], zzd[b], dd[b] = z[b, :kb + 1], zd[b, :kb], d[b, :kb]
        t0 = int(rs[b])
        g = oracle.accept_greedy(zz, dd)
        assert gr.accepted_len[b] == g.accepted_len[b]
        np.testing.assert_array_equal(gr.out_tokens[t0:t0 + kb + 1], g.out_tokens[b])
        s = oracle.accept_sample(zz, zzd, dd, T, seeds)
        assert sr.accepted_len[b] == s.accepted_len[b]
        np.testing.assert_array_equal(sr.out_tokens[t0:t0 + kb + 1], s.out_tokens[b])
        np.testing.assert_array_equal(sr.probs_at_draft[t0 - b:t0 - b + kb], s.probs_at_draft[b])


def test_zero_drafts_closed_form():
    B, V, T = 5, 400, 1.3
    counts = np.zeros(B, np.int32)
    _, z, _, _, seeds = _batch(B, 0, V, 21, counts=counts)
    rs = synth.row_start(counts)
    zp = z[:, 0]
    gr = oracle.accept_greedy_ragged(zp, None, rs, 4)
    np.testing.assert_array_equal(gr.accepted_len, 0)
    np.testing.assert_array_equal(gr.out_tokens, np.argmax(zp, axis=-1))
    sr = oracle.accept_sample_ragged(zp, None, None, rs, 4, T, seeds)
    np.testing.assert_array_equal(sr.accepted_len, 0)
    for b in range(B):
        _, u2 = oracle.verify_uniforms(np.array([seeds[b]]), np.array([b]), np.array([0]))
        x = zp[b] / T
        q = np.exp(x - x.max())
        C = np.cumsum(q)
        t = int(np.searchsorted(C, u2[0] * C[-1], side="right"))
        assert sr.out_tokens[b] == t


def test_malformed_offsets_mark_only_their_sequences():
    B, K_max, V = 5, 3, 100
    counts, z, zd, d, seeds = _batch(B, K_max, V, 8, counts=[1, 2, 0, 3, 1])
    rs, zp, zdp, dp = _packed(counts, z, zd, d)
    good = oracle.accept_sample_ragged(zp, zdp, dp, rs, K_max, 1.0, seeds)
    bad_rs = rs.copy()
    bad_rs[2] = bad_rs[3] + 1             # K_1 grows past sequence 2's start, K_2 = -2
    r = oracle.accept_sample_ragged(zp, zdp, dp, bad_rs, K_max, 1.0, seeds)
    assert r.accepted_len[1] == -1 and r.accepted_len[2] == -1   # K_1 = 4 > K_max, K_2 = -2
    np.testing.assert_array_equal(r.accepted_len[[0, 3, 4]], good.accepted_len[[0, 3, 4]])
    # K_b above K_max, and a last sequence that overruns the declared rows
    assert oracle.accept_greedy_ragged(zp, dp, rs, 2).accepted_len[3] == -1
    short = oracle.ragged_sequences(rs, int(rs[-1]) - 1, K_max)
    assert not short[-1][2] and all(ok for _, _, ok in short[:-1])
