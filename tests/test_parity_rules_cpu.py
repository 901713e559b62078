"""The GPU parity checkers themselves, on the CPU: they must pass outputs
equal to the oracle's, count near-ties per decision type, and fail the
mistakes a selection or acceptance bug would make (a terminal token one
step or one 4096-entry chunk away, an accept decision or a greedy token
flipped at a clear margin), while letting a flip through only where the
rounding bound allows it and u'Z sits within that bound of the GPU token's
CDF step.  Outputs here come from the oracle, with planted changes.
"""
import numpy as np
import pytest

import oracle
from gpu_support import Tally, row_bounds, sample_bound_ctx, strict_greedy, strict_sample, terminal_bound


def _case(B=24, K=4, V=9000, T=0.9, seed=3):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1.3, (B, K + 1, V))
    zd = z[:, :K] + rng.normal(0, 0.5, (B, K, V))
    p = oracle.softmax(zd, T)
    d = np.array([[rng.choice(V, p=p[b, i]) for i in range(K)] for b in range(B)], np.int32)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(77)
    probs = oracle.sample_probs(z, zd, d, T)
    res = oracle.accept_sample_probs(probs, d, seeds)
    return z, zd, d, T, seeds, probs, res


def test_equal_outputs_pass_and_are_counted():
    z, zd, d, T, seeds, probs, res = _case()
    ctx = sample_bound_ctx(probs, z, zd, T)
    t = strict_sample(res, res.accepted_len, res.out_tokens, range(len(d)), ctx, d)
    assert t.rows == len(d) and t.types["terminal"].decisions == len(d)
    assert t.types["accept"].decisions >= len(d)
    assert all(t.types[k].flips == 0 for k in t.types)
    # at V = 9000 terminal margins are far above the bound for most draws
    tt = t.types["terminal"]
    assert tt.below_bound < tt.decisions


def test_one_call_equals_decisions_on_its_probabilities():
    """accept_sample is sample_probs followed by accept_sample_probs, and many
    rounds of one sequence can be checked as one broadcast batch."""
    z, zd, d, T, seeds, probs, res = _case(B=6)
    ref = oracle.accept_sample(z, zd, d, T, seeds)
    for f in ("accepted_len", "out_tokens", "terminal_margin", "accept_margin"):
        np.testing.assert_array_equal(getattr(ref, f), getattr(res, f))
    one = oracle.sample_probs(z[:1], zd[:1], d[:1], T)
    R = 5
    bc = oracle.SampleProbs(R, one.K, one.V, np.arange(R), np.zeros(0, np.int64),
                            np.broadcast_to(one.q, (R,) + one.q.shape[1:]),
                            np.broadcast_to(one.p, (R,) + one.p.shape[1:]),
                            np.broadcast_to(one.alpha, (R,) + one.alpha.shape[1:]))
    dr = np.repeat(d[:1], R, axis=0)
    sr = np.arange(R, dtype=np.uint64) + np.uint64(500)
    got = oracle.accept_sample_probs(bc, dr, sr, slots=np.zeros(R, np.int64))
    for r in range(R):
        want = oracle.accept_sample(z[:1], zd[:1], d[:1], T, sr[r:r + 1])
        assert got.accepted_len[r] == want.accepted_len[0]
        assert np.array_equal(got.out_tokens[r], want.out_tokens[0])


def _first_draw(res, K, margin_at_least):
    for b in range(len(res.accepted_len)):
        if res.terminal_margin[b] >= margin_at_least:
            return b
    raise AssertionError("no draw with such a margin")


@pytest.mark.parametrize("shift", [1, -1, 4096])
def test_wrong_terminal_token_fails(shift):
    z, zd, d, T, seeds, probs, res = _case()
    K, V = d.shape[1], z.shape[-1]
    ctx = sample_bound_ctx(probs, z, zd, T)
    b = _first_draw(res, K, 1e-3)
    out = res.out_tokens.copy()
    n = res.accepted_len[b]
    out[b, n] = (out[b, n] + shift) % V
    with pytest.raises(AssertionError):
        strict_sample(res, res.accepted_len, out, range(len(d)), ctx, d)


def test_flipped_accept_decision_fails():
    z, zd, d, T, seeds, probs, res = _case()
    K = d.shape[1]
    ctx = sample_bound_ctx(probs, z, zd, T)
    b = next(b for b in range(len(d)) if res.accepted_len[b] < K and res.accept_margin[b, res.accepted_len[b]] > 1e-2)
    acc = res.accepted_len.copy()
    out = res.out_tokens.copy()
    n = acc[b]
    acc[b] = n + 1                 # the GPU "accepted" the draft the oracle rejected
    out[b, n] = d[b, n]
    with pytest.raises(AssertionError):
        strict_sample(res, acc, out, range(len(d)), ctx, d)


def test_greedy_flip_fails_on_same_logits_and_passes_within_deviation():
    rng = np.random.default_rng(5)
    B, K, V = 16, 4, 500
    z = rng.normal(0, 1, (B, K + 1, V))
    d = np.argmax(z[:, :K], axis=-1).astype(np.int32)
    d[:, 2] = (d[:, 2] + 1) % V
    res = oracle.accept_greedy(z, d)
    out = res.out_tokens.copy()
    b = 0
    n = res.accepted_len[b]
    # the runner-up token at the decided position
    second = int(np.argsort(-z[b, n])[1])
    out[b, n] = second
    with pytest.raises(AssertionError):
        strict_greedy(res, res.accepted_len, out, range(B), delta=None)
    # with a logit deviation of half the top1 - top2 gap the same flip is
    # explained (the margin is below 2 delta) -- but only below 1e-4
    m = res.margin[b, n]
    delta = np.full(B, m)
    if m < 1e-4:
        t = strict_greedy(res, res.accepted_len, out, range(B), delta=delta)
        assert t.types["greedy"].flips == 1
    else:
        with pytest.raises(AssertionError):
            strict_greedy(res, res.accepted_len, out, range(B), delta=delta)


def test_terminal_flip_within_bound_is_counted():
    """A terminal draw that lands next to a CDF step may flip to the
    neighbouring token when the rounding bound covers the distance."""
    z, zd, d, T, seeds, probs, res = _case(V=200000, B=40)
    K, V = d.shape[1], z.shape[-1]
    # end-to-end mode with a large logit deviation makes the bound cover the
    # step next to the draw
    delta = np.full((len(d), K + 1), 2e-5)
    ctx = sample_bound_ctx(probs, z, zd, T, delta=delta)
    t = Tally()
    for b in range(len(d)):
        n = res.accepted_len[b]
        if res.terminal_margin[b] >= 1e-4:
            continue
        j = list(probs.good).index(b)
        bonus = n == K
        bound = terminal_bound(ctx.tq, None if bonus else ctx.tp, 0.0 if bonus else probs.alpha[j, n],
                               res.residual_mass[b], (j, n), None if bonus else (j, n), 2e-5, T)
        if res.terminal_margin[b] >= bound:
            continue
        # the neighbour across the nearer step
        q = probs.q[j, n]
        w = q if bonus else oracle.verify.terminal_weights(q, probs.p[j, n])
        C = np.cumsum(w)
        x = res.u_terminal[b, n] * C[-1]
        tok = res.out_tokens[b, n]
        lo = C[tok - 1] if tok > 0 else 0.0
        nb = tok - 1 if x - lo < C[tok] - x else tok + 1
        while 0 <= nb < V and w[nb] == 0:
            nb += 1 if nb > tok else -1
        if not 0 <= nb < V:
            continue
        out = res.out_tokens.copy()
        out[b, n] = nb
        strict_sample(res, res.accepted_len, out, [b], ctx, d, t)
        break
    else:
        pytest.skip("no draw close enough to a step in this sample")
    assert t.types["terminal"].flips == 1
    assert 0 < t.types["terminal"].max_flip_consistency <= 1


def test_bounds_are_positive_and_small():
    z, zd, d, T, seeds, probs, res = _case()
    rb = row_bounds(z[probs.good], probs.q, T)
    assert np.all(rb.spec > 0) and np.all(rb.common > 0)
    assert np.all(rb.spec < 1e-4) and np.all(rb.common < 1e-4)


def test_flip_below_stated_tolerance_but_above_bound_fails():
    """The stricter rule has power where the 1e-4 rule has none: at a large
    vocabulary a draw with margin between the rounding bound and 1e-4 must
    still match exactly."""
    z, zd, d, T, seeds, probs, res = _case(V=200000, B=40)
    K, V = d.shape[1], z.shape[-1]
    ctx = sample_bound_ctx(probs, z, zd, T)
    for b in range(len(d)):
        n = res.accepted_len[b]
        j = list(probs.good).index(b)
        bonus = n == K
        bound = terminal_bound(ctx.tq, None if bonus else ctx.tp, 0.0 if bonus else probs.alpha[j, n],
                               res.residual_mass[b], (j, n), None if bonus else (j, n), 0.0, T)
        if bound <= res.terminal_margin[b] < 1e-4:
            out = res.out_tokens.copy()
            out[b, n] = (out[b, n] + 1) % V
            with pytest.raises(AssertionError, match="rounding bound"):
                strict_sample(res, res.accepted_len, out, [b], ctx, d)
            return
    pytest.skip("no draw with a margin between the bound and 1e-4 in this sample")
