"""Pins for the oracle's speculative sampling (accept test, residual and bonus
draws, expected tokens per pass).

What the pages fix, and the test that checks it:
* The output is distributed exactly as the target ("Inference-4", sampling
  bullet; "speculative-decoding" blog, Rejection sampling; "Speculative
  decoding" course page, Why this is not approximate): chi-square over 10^6
  verify rounds, per position, against softmax(z/T) from scipy.  The drafts
  must be sampled from the draft distribution; argmax drafts must fail the
  same test (negative control: the test has power).
* Accepted overlap plus resampled leftover mass rebuild the target exactly
  (blog, Rejection sampling): exact enumeration over every draft token and a
  fine grid of terminal uniforms.
* A token the target likes at least as much as the draft is always accepted
  ("What is speculative decoding" guide, How speculative decoding works):
  p = q accepts every draft.
* E[tokens per pass] = (1 - a^(K+1)) / (1 - a), limits 1 and K+1, and the
  guide's worked example (~2.8 at gamma=4, a=0.7): Monte Carlo with
  constructed constant-acceptance pairs.
"""
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle.verify as ov
from oracle.verify import (accept_ratio, accept_sample, expected_tokens,
                           expected_tokens_positional, inverse_cdf, terminal_weights)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _chisq_pvalue(observed_tokens, probs):
    """Chi-square goodness of fit, bins with expected count < 5 merged."""
    V = len(probs)
    obs = np.bincount(observed_tokens, minlength=V).astype(np.float64)
    exp = probs * obs.sum()
    order = np.argsort(exp)
    small = exp[order] < 5
    o = list(obs[order][~small])
    e = list(exp[order][~small])
    if small.any():
        o.append(obs[order][small].sum())
        e.append(exp[order][small].sum())
    o, e = np.array(o), np.array(e)
    keep = e > 0
    assert np.all(o[~keep] == 0), "token drawn with zero target probability"
    return stats.chisquare(o[keep], e[keep] * o[keep].sum() / e[keep].sum()).pvalue


def _run_rounds(zt, zd, T, n_rounds, draft_mode="sample", chunk=100_000, seed0=0):
    """Run n_rounds verify rounds with fixed logits (one row per round, seeds
    seed0 + r), drafts redrawn each round by the test's own sampler."""
    P, V = zt.shape
    K = P - 1
    pd = special.softmax(zd / T, axis=-1) if K else np.zeros((0, V))
    rng = np.random.default_rng(99)
    acc, tok = [], []
    for r0 in range(0, n_rounds, chunk):
        R = min(chunk, n_rounds - r0)
        if draft_mode == "sample":
            d = np.stack([rng.choice(V, size=R, p=pd[i]) for i in range(K)], -1) if K else np.zeros((R, 0), int)
        else:
            d = np.broadcast_to(np.argmax(zd, -1), (R, K)).copy()
        res = accept_sample(np.broadcast_to(zt, (R, P, V)), np.broadcast_to(zd, (R, K, V)), d, T,
                            np.arange(seed0 + r0, seed0 + r0 + R, dtype=np.uint64))
        acc.append(res.accepted_len)
        tok.append(res.out_tokens)
    return np.concatenate(acc), np.concatenate(tok)


def _position_pvalues(acc, tok, q):
    K = q.shape[0] - 1
    pv = []
    for i in range(K + 1):
        reached = acc >= i
        pv.append(_chisq_pvalue(tok[reached, i], q[i]))
    return pv


@pytest.mark.slow
def test_chisquare_1e6_rounds_matches_target():
    rng = np.random.default_rng(2024)
    K, V, T = 3, 32, 1.0
    zt = rng.normal(size=(K + 1, V)) * 1.5
    zd = zt[:K] + rng.normal(size=(K, V))
    acc, tok = _run_rounds(zt, zd, T, 1_000_000)
    q = special.softmax(zt / T, axis=-1)
    pv = _position_pvalues(acc, tok, q)
    assert min(pv) > 1e-3, pv
    # the run visits every branch: rejections at each position and bonus tokens
    assert set(np.unique(acc)) == set(range(K + 1))


def test_chisquare_temperature():
    rng = np.random.default_rng(11)
    K, V, T = 2, 24, 0.7
    zt = rng.normal(size=(K + 1, V))
    zd = 0.7 * zt[:K] + rng.normal(size=(K, V))
    acc, tok = _run_rounds(zt, zd, T, 200_000, seed0=10_000_000)
    pv = _position_pvalues(acc, tok, special.softmax(zt / T, axis=-1))
    assert min(pv) > 1e-3, pv


def test_negative_control_argmax_drafts_fail():
    rng = np.random.default_rng(2024)
    K, V, T = 3, 32, 1.0
    zt = rng.normal(size=(K + 1, V)) * 1.5
    zd = zt[:K] + rng.normal(size=(K, V))
    acc, tok = _run_rounds(zt, zd, T, 100_000, draft_mode="argmax")
    assert _chisq_pvalue(tok[:, 0], special.softmax(zt[0] / T)) < 1e-9


def test_k0_bonus_is_target_sample():
    rng = np.random.default_rng(5)
    V = 40
    zt = rng.normal(size=(1, V))
    acc, tok = _run_rounds(zt, np.zeros((0, V)), 1.0, 100_000)
    assert np.all(acc == 0)
    assert _chisq_pvalue(tok[:, 0], special.softmax(zt[0])) > 1e-3


def test_exact_enumeration_rebuilds_target():
    """sum_d p(d) [r(d) 1{y=d} + (1 - r(d)) P_term(y)] = q(y), with P_term the
    law of the oracle's terminal draw measured on a 2^16-point uniform grid."""
    rng = np.random.default_rng(6)
    grid = (np.arange(2 ** 16) + 0.5) / 2 ** 16
    for trial in range(20):
        V = int(rng.integers(2, 14))
        q = special.softmax(rng.normal(size=V) * 2)
        p = special.softmax(rng.normal(size=V) * 2)
        if trial == 0:
            q[0], q[1:] = 0.0, q[1:] / q[1:].sum()      # a token the target rules out
        r = accept_ratio(q, p)
        # probability of accepting = overlap mass
        np.testing.assert_allclose(np.sum(p * r), np.sum(np.minimum(p, q)), rtol=0, atol=1e-12)
        w = terminal_weights(q, p)
        t, _, _ = inverse_cdf(np.broadcast_to(w, (len(grid), V)), grid)
        p_term = np.bincount(t, minlength=V) / len(grid)
        emit = p * r + (1.0 - np.sum(p * r)) * p_term
        np.testing.assert_allclose(emit, q, rtol=0, atol=4 * V * 2.0 ** -16)
        assert np.all(p_term[q == 0] == 0)


def test_accept_ratio_special_cases():
    r = accept_ratio(np.array([0.2, 0.4, 0.0, 0.5, 0.0, 0.3]), np.array([0.4, 0.2, 0.0, 0.0, 0.3, 0.3]))
    assert r.tolist() == [0.5, 1.0, 0.0, 1.0, 0.0, 1.0]


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(7)
    K, V = 4, 30
    zt = rng.normal(size=(K + 1, V))
    acc, tok = _run_rounds(zt, zt[:K].copy(), 1.0, 20_000)
    assert np.all(acc == K)


def test_disjoint_supports_reject_at_once():
    rng = np.random.default_rng(8)
    K, V = 3, 20
    zt = rng.normal(size=(K + 1, V))
    zd = rng.normal(size=(K, V))
    zt[:, 10:] = -np.inf               # target lives on tokens 0..9
    zd[:, :10] = -np.inf               # draft lives on tokens 10..19
    acc, tok = _run_rounds(zt, zd, 1.0, 20_000)
    assert np.all(acc == 0)
    assert np.all(tok[:, 0] < 10)


def _constant_alpha_pair(rng, V, alpha):
    """Target q on tokens 0..V-2 and a sink token V-1 with target logit -1e4
    (probability exactly 0 in fp64); draft p = alpha*q on the support and
    1-alpha on the sink.  Non-sink drafts have r = 1, the sink has r = 0, so
    each draft is accepted with probability alpha exactly."""
    zt = np.append(rng.normal(size=V - 1), -1e4)
    q = special.softmax(zt)
    assert q[-1] == 0.0
    p = np.append(alpha * q[:-1], 1.0 - alpha)
    with np.errstate(divide="ignore"):
        zd = np.log(p)
    return zt, zd


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.7, 0.9, 1.0])
def test_expected_tokens_monte_carlo(alpha):
    rng = np.random.default_rng(int(alpha * 10) + 1)
    K, V, N = 4, 16, 100_000
    pairs = [_constant_alpha_pair(rng, V, alpha) for _ in range(K + 1)]
    zt = np.stack([a for a, _ in pairs])
    zd = np.stack([b for _, b in pairs[:K]])
    acc, tok = _run_rounds(zt, zd, 1.0, N, seed0=int(alpha * 1e7))
    tokens = acc + 1.0
    se = tokens.std(ddof=1) / np.sqrt(N) if tokens.std() > 0 else 0.0
    assert abs(tokens.mean() - expected_tokens(alpha, K)) <= 4 * se + 1e-12
    # each reached position accepts with probability alpha
    for i in range(K):
        reached = acc >= i
        if reached.sum() > 1000:
            frac = np.mean(acc[reached] > i)
            assert abs(frac - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / reached.sum()) + 1e-12


def test_expected_tokens_closed_form_and_worked_example():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "expected_tokens_worked_example.txt"))
            if ln.strip() and not ln.startswith("#")]
    for gamma, alpha, printed, prec in rows:
        got = expected_tokens(float(alpha), int(gamma))
        assert abs(got - float(printed)) <= float(prec)
    # the blog's form: a finite geometric sum
    for a in [0.0, 0.1, 0.5, 0.7, 0.99, 1.0]:
        for K in [0, 1, 4, 8]:
            assert expected_tokens(a, K) == pytest.approx(sum(a ** i for i in range(K + 1)), abs=1e-12)
    assert expected_tokens(1.0, 4) == 5.0
    assert expected_tokens(0.0, 4) == 1.0
    assert expected_tokens_positional([0.5, 0.5]) == pytest.approx(expected_tokens(0.5, 2))


def test_positional_acceptance_general_pairs():
    """Drafts from p: P(accept at i | reached i) = sum_v min(q_i, p_i)."""
    rng = np.random.default_rng(21)
    K, V, N = 4, 20, 200_000
    zt = rng.normal(size=(K + 1, V)) * 1.2
    zd = zt[:K] + rng.normal(size=(K, V)) * np.array([0.3, 0.8, 1.5, 3.0])[:, None]
    acc, tok = _run_rounds(zt, zd, 1.0, N, seed0=5_000_000)
    q = special.softmax(zt, axis=-1)
    p = special.softmax(zd, axis=-1)
    alphas = np.sum(np.minimum(q[:K], p), axis=-1)
    for i in range(K):
        reached = acc >= i
        frac = np.mean(acc[reached] > i)
        assert abs(frac - alphas[i]) < 4 * np.sqrt(alphas[i] * (1 - alphas[i]) / reached.sum())
    tokens = acc + 1.0
    assert abs(tokens.mean() - expected_tokens_positional(alphas)) < 4 * tokens.std() / np.sqrt(N)


def test_probs_at_draft_and_alpha_outputs():
    rng = np.random.default_rng(9)
    B, K, V, T = 3, 2, 15, 0.8
    zt = rng.normal(size=(B, K + 1, V))
    zd = rng.normal(size=(B, K, V))
    d = rng.integers(0, V, size=(B, K))
    res = accept_sample(zt, zd, d, T, np.arange(B, dtype=np.uint64))
    q = special.softmax(zt / T, axis=-1)
    p = special.softmax(zd / T, axis=-1)
    for b in range(B):
        for i in range(K):
            assert res.probs_at_draft[b, i, 0] == pytest.approx(q[b, i, d[b, i]], rel=1e-12)
            assert res.probs_at_draft[b, i, 1] == pytest.approx(p[b, i, d[b, i]], rel=1e-12)
            assert res.alpha[b, i] == pytest.approx(np.minimum(q[b, i], p[b, i]).sum(), rel=1e-12)


def test_inverse_cdf_margin_property():
    """Moving the draw point by less than margin*Z keeps the token; moving it
    just past the nearer CDF step changes it."""
    rng = np.random.default_rng(10)
    for _ in range(200):
        V = int(rng.integers(2, 30))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            continue
        u = rng.random()
        t, Z, m = inverse_cdf(w, u)
        assert w[t] > 0 and m >= 0
        C = np.cumsum(w)
        x = u * Z
        for dx in (0.999 * m * Z, -0.999 * m * Z):
            if 0 <= x + dx < Z:
                assert inverse_cdf(w, (x + dx) / Z)[0] == t
        lo = C[t - 1] if t > 0 else 0.0
        if x - lo < C[t] - x and t > 0:
            assert inverse_cdf(w, (lo - 1e-9 * Z) / Z)[0] != t
        elif C[t] < Z * (1 - 1e-9):        # a later token still carries mass
            assert inverse_cdf(w, (C[t] + 1e-12 * Z) / Z)[0] != t


def test_bad_rows_and_subset():
    rng = np.random.default_rng(12)
    B, K, V = 5, 2, 9
    zt = rng.normal(size=(B, K + 1, V))
    zd = rng.normal(size=(B, K, V))
    d = rng.integers(0, V, size=(B, K))
    d[1, 1] = -1
    zd[2, 0, 4] = np.inf
    zt[3, 2] = -np.inf
    res = accept_sample(zt, zd, d, 1.0, np.arange(B, dtype=np.uint64), rows=[0, 1, 2, 3])
    assert res.accepted_len[1:].tolist() == [-1, -1, -1, -2]
    assert res.accepted_len[0] >= 0
    assert np.all(res.out_tokens[1:] == -1)


def test_inverse_cdf_never_draws_zero_weight():
    """A token with zero weight is never drawn, also at u = 0 and when u*Z
    lands exactly on a CDF step (both occur on the 24-bit uniform grid)."""
    w = np.array([0.0, 0.0, 1.0, 0.0, 1.0, 2.0, 0.0])
    assert inverse_cdf(w, 0.0)[0] == 2
    assert inverse_cdf(w, 0.25)[0] == 4          # uZ = 1 = C_2 = C_3 exactly
    assert inverse_cdf(w, 0.5)[0] == 5           # uZ = 2 = C_4 exactly
    assert inverse_cdf(w, 1 - 2.0 ** -24)[0] == 5
    grid = np.arange(2 ** 12) / 2 ** 12          # includes 0 and exact steps
    t, _, _ = inverse_cdf(np.broadcast_to(w, (len(grid), len(w))), grid)
    assert np.all(w[t] > 0)


@pytest.mark.parametrize("K", [0, 1, 4])
def test_rounds_form_equals_round_by_round(K):
    """accept_sample_rounds (terminal CDFs formed once, draws looked up) gives
    field for field what accept_sample_probs gives round by round, faulted
    rows, residuals without mass and bonus draws included."""
    rng = np.random.default_rng(40 + K)
    B, V, T, R = 7, 300, 0.8, 12
    z = rng.normal(0, 2, (B, K + 1, V))
    zd = z[:, :K] + rng.normal(0, 0.7, (B, K, V))
    if K:
        zd[1] = z[1, :K]                       # p = q: every draft accepted, bonus draws
        zd[2, 0, :] = z[2, 0, :]               # residual without mass at position 0
    z[3, 0, 5] = np.nan                        # a faulted row
    d = rng.integers(0, V, (R, B, K))
    seeds = rng.integers(0, 2**63, (R, B)).astype(np.uint64)
    probs = ov.sample_probs(z, zd, d[0], T, rows=[0, 1, 2, 3, 4, 6])
    got = ov.accept_sample_rounds(probs, d, seeds)
    for r in range(R):
        want = ov.accept_sample_probs(probs, d[r], seeds[r])
        for f in ("accepted_len", "out_tokens", "probs_at_draft", "ratio", "u_accept", "u_terminal",
                  "accept_margin", "terminal_margin", "residual_mass", "alpha"):
            np.testing.assert_array_equal(getattr(got, f)[r], getattr(want, f), err_msg="%s round %d" % (f, r))
