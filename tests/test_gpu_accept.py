"""GPU parity of spec_accept_greedy / spec_accept_sample against the oracle,
with the target and draft logits given as fp32 inputs (no LM head), so both
sides decide on identical values: greedy rows must agree exactly, sampled
rows decision by decision with near-ties counted.

Covers K = 0 (plain argmax / bonus draw), K = 63 (the largest K one
wavefront scans), V not a multiple of 4 (unaligned rows: scalar loads), V
spanning many chunks with a ragged last one, argmax ties, row subsets and a
mixed greedy/sampled batch over one logits buffer, data-fault rows, and the
accept-ratio edge cases (draft or target probability exactly zero).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import (PROB_ATOL, ParityCounts, compare_greedy, compare_sample, dev, gpu_accept_greedy,
                         gpu_accept_sample, say)

pytestmark = pytest.mark.gpu


def _logits(B, K, V, seed, scale=2.0, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    zt = torch.randn((B, K + 1, V), generator=g) * scale
    noise = torch.randn((B, K, V), generator=g) * sigma
    zd = zt[:, :K] + noise
    return zt, zd


def _sampled_drafts(zd, T, seed):
    B, K, V = zd.shape
    if K == 0:
        return torch.zeros((B, 0), dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    u = torch.rand((B, K, V), generator=g, dtype=torch.float64).clamp_(min=1e-300)
    return torch.argmax(zd.double() / T - torch.log(-torch.log(u)), dim=-1).to(torch.int32)


def _greedy_drafts(zt, seed, p_keep=0.8):
    """Drafts equal to the target argmax, each corrupted with prob 1-p_keep,
    so accepted lengths spread over 0..K."""
    B, P, V = zt.shape
    K = P - 1
    if K == 0:
        return torch.zeros((B, 0), dtype=torch.int32)
    g = torch.Generator().manual_seed(seed)
    a = torch.argmax(zt[:, :K], dim=-1)
    bad = torch.rand((B, K), generator=g) > p_keep
    other = torch.randint(0, V, (B, K), generator=g)
    return torch.where(bad, other, a).to(torch.int32)


@pytest.mark.parametrize("K", [0, 1, 4, 63])
@pytest.mark.parametrize("V", [1000, 5003, 2 * 4096 + 7])
def test_greedy_exact(K, V):
    B = 96
    say("greedy exact B=%d K=%d V=%d" % (B, K, V))
    zt, _ = _logits(B, K, V, seed=K * 1000 + V)
    zt[::7, :, 3] = zt[::7].max(dim=-1).values       # ties with the max: lowest index must win
    zt[::11, :, V - 1] = zt[::11].max(dim=-1).values
    d = _greedy_drafts(zt, seed=V)
    acc, out = gpu_accept_greedy(zt.to(dev()), d.to(dev()))
    res = oracle.accept_greedy(zt.numpy(), d.numpy())
    c = compare_greedy(res, acc.cpu().numpy(), out.cpu().numpy(), range(B), exact=True)
    say("  " + str(c) + " accepted=%s" % np.bincount(acc.cpu().numpy(), minlength=K + 1).tolist())


@pytest.mark.parametrize("K,T", [(0, 1.0), (3, 1.0), (8, 0.7), (63, 1.3)])
@pytest.mark.parametrize("V", [1000, 5003, 3 * 4096 + 1])
def test_sample_parity(K, T, V):
    B = 128
    say("sampled parity B=%d K=%d V=%d T=%g" % (B, K, V, T))
    zt, zd = _logits(B, K, V, seed=K * 31 + V, scale=1.5, sigma=0.8)
    d = _sampled_drafts(zd, T, seed=V + K)
    seeds = np.arange(B, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(V)
    acc, out, pad = gpu_accept_sample(zt.to(dev()), zd.to(dev()), d.to(dev()), T, seeds, probs=True)
    res = oracle.accept_sample(zt.numpy(), zd.numpy(), d.numpy(), T, seeds)
    c = compare_sample(res, acc.cpu().numpy(), out.cpu().numpy(), range(B))
    say("  " + str(c) + " accepted=%s" % np.bincount(acc.cpu().numpy(), minlength=K + 1).tolist())
    if K:
        np.testing.assert_allclose(pad.cpu().numpy(), res.probs_at_draft, rtol=0, atol=PROB_ATOL)


def test_mixed_batch_and_row_subsets():
    """Greedy rows and sampled rows verified by two calls over one logits
    buffer; rows in neither list keep their previous contents."""
    B, K, V, T = 40, 4, 3001, 0.8
    zt, zd = _logits(B, K, V, seed=5)
    rng = np.random.default_rng(0)
    perm = rng.permutation(B)
    greedy_rows, sampled_rows = np.sort(perm[:15]), perm[15:32]      # rows perm[32:] untouched
    d = _sampled_drafts(zd, T, seed=6)
    d[greedy_rows] = _greedy_drafts(zt, seed=7)[greedy_rows]
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(1 << 33)
    ztd, zdd, dd = zt.to(dev()), zd.to(dev()), d.to(dev())
    acc, out = gpu_accept_greedy(ztd, dd, rows=greedy_rows)
    acc, out, _ = gpu_accept_sample(ztd, zdd, dd, T, seeds, rows=sampled_rows, acc=acc, out=out)
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    rg = oracle.accept_greedy(zt.numpy(), d.numpy(), rows=greedy_rows)
    rs = oracle.accept_sample(zt.numpy(), zd.numpy(), d.numpy(), T, seeds, rows=sampled_rows)
    c = compare_greedy(rg, acc, out, greedy_rows, exact=True).merge(compare_sample(rs, acc, out, sampled_rows))
    say("mixed batch: " + str(c))
    untouched = perm[32:]
    assert np.all(acc[untouched] == -2) and np.all(out[untouched] == -9)


def test_fault_rows_marked():
    B, K, V, T = 12, 3, 777, 1.0
    zt, zd = _logits(B, K, V, seed=9)
    d = _sampled_drafts(zd, T, seed=10)
    d[1, 2] = V              # out of range
    d[2, 0] = -1
    zt[3, 3, 5] = float("nan")      # NaN in the bonus row
    zt[4, 0, 9] = float("inf")
    zt[5, 1, :] = float("-inf")     # no finite logit
    zd[6, 2, :] = float("-inf")     # draft row with no finite logit (sampled only)
    zd[7, 0, 100] = float("nan")    # NaN in a draft row (sampled only)
    seeds = np.arange(B, dtype=np.uint64)
    ztd, zdd, dd = zt.to(dev()), zd.to(dev()), d.to(dev())
    acc_s, out_s, _ = gpu_accept_sample(ztd, zdd, dd, T, seeds)
    rs = oracle.accept_sample(zt.numpy(), zd.numpy(), d.numpy(), T, seeds)
    c = compare_sample(rs, acc_s.cpu().numpy(), out_s.cpu().numpy(), range(B))
    assert c.faulted == 7, c
    acc_g, out_g = gpu_accept_greedy(ztd, dd)
    rg = oracle.accept_greedy(zt.numpy(), d.numpy())
    cg = compare_greedy(rg, acc_g.cpu().numpy(), out_g.cpu().numpy(), range(B), exact=True)
    assert cg.faulted == 5, cg
    say("faults: sampled %s | greedy %s" % (c, cg))


def test_zero_probability_edges():
    """Draft token impossible under the target -> rejected; impossible under
    the draft but possible under the target -> accepted; the redraw never
    lands on a token the target rules out."""
    B, K, V = 64, 2, 50
    g = torch.Generator().manual_seed(11)
    zt = torch.randn((B, K + 1, V), generator=g)
    zd = torch.randn((B, K, V), generator=g)
    d = torch.randint(0, V, (B, K), generator=g).to(torch.int32)
    for b in range(0, B, 2):
        zt[b, 0, d[b, 0]] = float("-inf")       # target rules the first draft out
        zt[b, 0, 40:] = float("-inf")
    for b in range(1, B, 2):
        zd[b, 0, d[b, 0]] = float("-inf")       # draft would never have proposed it
    seeds = np.arange(B, dtype=np.uint64) * np.uint64(977)
    acc, out, pad = gpu_accept_sample(zt.to(dev()), zd.to(dev()), d.to(dev()), 1.0, seeds, probs=True)
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    res = oracle.accept_sample(zt.numpy(), zd.numpy(), d.numpy(), 1.0, seeds)
    compare_sample(res, acc, out, range(B))
    assert np.all(acc[0::2] == 0) and np.all(out[0::2, 0] < 40)
    assert np.all(acc[1::2] >= 1)
    np.testing.assert_allclose(pad.cpu().numpy(), res.probs_at_draft, rtol=0, atol=PROB_ATOL)


def test_single_token_vocabulary():
    B, K, V = 5, 3, 1
    zt = torch.zeros((B, K + 1, V))
    zd = torch.zeros((B, K, V))
    d = torch.zeros((B, K), dtype=torch.int32)
    ztd, zdd, dd = zt.to(dev()), zd.to(dev()), d.to(dev())
    acc, out = gpu_accept_greedy(ztd, dd)
    assert np.all(acc.cpu().numpy() == K) and np.all(out.cpu().numpy() == 0)
    acc, out, _ = gpu_accept_sample(ztd, zdd, dd, 1.0, np.arange(B, dtype=np.uint64))
    assert np.all(acc.cpu().numpy() == K) and np.all(out.cpu().numpy() == 0)


def test_accept_deterministic():
    B, K, V, T = 32, 5, 20011, 0.9
    zt, zd = _logits(B, K, V, seed=12)
    d = _sampled_drafts(zd, T, seed=13)
    seeds = np.arange(B, dtype=np.uint64)
    ztd, zdd, dd = zt.to(dev()), zd.to(dev()), d.to(dev())
    r1 = gpu_accept_sample(ztd, zdd, dd, T, seeds, probs=True)
    r2 = gpu_accept_sample(ztd, zdd, dd, T, seeds, probs=True)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("V", [5003, 2 * 4096 + 7])
def test_fused_accept_residual_matches_two_kernels(V):
    """Small sampled batches run acceptance and the residual draw in one
    launch (sequences x (2K+1) <= 48 rows), larger ones in two.  Four
    sequences at K = 5 (44 rows) take the fused launch; the same four plus a
    fifth (55 rows) take the two kernels: the four must come out identical,
    and both must meet the oracle."""
    B, K, T = 5, 5, 0.9
    zt, zd = _logits(B, K, V, seed=V + 11)
    d = _sampled_drafts(zd, T, seed=V)
    seeds = np.arange(B, dtype=np.uint64) * 7919 + 3
    say("fused vs two-kernel accept + residual, V=%d" % V)
    acc_f, out_f, pad_f = gpu_accept_sample(zt.to(dev()), zd.to(dev()), d.to(dev()), T, seeds, rows=[0, 1, 2, 3],
                                            probs=True)
    acc_s, out_s, pad_s = gpu_accept_sample(zt.to(dev()), zd.to(dev()), d.to(dev()), T, seeds,
                                            rows=[0, 1, 2, 3, 4], probs=True)
    acc_f, out_f, acc_s, out_s = acc_f.cpu().numpy(), out_f.cpu().numpy(), acc_s.cpu().numpy(), out_s.cpu().numpy()
    np.testing.assert_array_equal(acc_f[:4], acc_s[:4])
    np.testing.assert_array_equal(out_f[:4], out_s[:4])
    np.testing.assert_array_equal(pad_f.cpu().numpy()[:4], pad_s.cpu().numpy()[:4])
    res = oracle.accept_sample(zt.double().numpy(), zd.double().numpy(), d.numpy(), T, seeds)
    c = compare_sample(res, acc_s, out_s, range(B))
    say("  " + str(c))


def test_largest_vocabulary():
    """V at the library's limit (1024 chunks of 4096: the residual keeps one
    prefix entry per chunk in LDS), both rules, against the oracle."""
    B, K, V, T = 2, 2, 1024 * 4096, 1.0
    g = torch.Generator().manual_seed(17)
    zt = torch.randn((B, K + 1, V), generator=g) * 3.0
    zd = zt[:, :K] + torch.randn((B, K, V), generator=g)
    d = _sampled_drafts(zd, T, seed=5)
    dg = _greedy_drafts(zt, seed=6)
    seeds = np.array([11, 12], dtype=np.uint64)
    say("largest vocabulary V=%d" % V)
    acc, out = gpu_accept_greedy(zt.to(dev()), dg.to(dev()))
    res = oracle.accept_greedy(zt.double().numpy(), dg.numpy())
    c = compare_greedy(res, acc.cpu().numpy(), out.cpu().numpy(), range(B), exact=True)
    acc, out, _ = gpu_accept_sample(zt.to(dev()), zd.to(dev()), d.to(dev()), T, seeds)
    res = oracle.accept_sample(zt.double().numpy(), zd.double().numpy(), d.numpy(), T, seeds)
    c.merge(compare_sample(res, acc.cpu().numpy(), out.cpu().numpy(), range(B)))
    say("  " + str(c))


@pytest.mark.parametrize("T", [0.05, 0.25, 4.0])
def test_sample_extreme_temperatures(T):
    """Very sharp and very flat distributions at full vocabulary.  At T = 0.05
    (logits of spread 2, so z/T spreads over ~40) almost every term of the
    softmax sums and residual weights underflows: the kernels flush
    probabilities below 2^-126 to zero, which moves a sum by less than its
    own rounding.  At T = 4 every one of the 128256 terms counts.  All
    sequences (statistics pass, counted residual), eight of them (polled
    residual) and one (acceptance and draw in one launch), each against the
    oracle by the margin rule, probabilities within PROB_ATOL."""
    B, K, V = 64, 4, 128256
    zt, zd = _logits(B, K, V, seed=int(T * 1000) + 7, scale=2.0, sigma=0.6)
    d = _sampled_drafts(zd, T, seed=int(T * 100) + 3)
    seeds = np.arange(B, dtype=np.uint64) * np.uint64(7919) + np.uint64(int(T * 100))
    res = oracle.accept_sample(zt.numpy(), zd.numpy(), d.numpy(), T, seeds)
    zt_d, zd_d, d_d = zt.to(dev()), zd.to(dev()), d.to(dev())
    for rows in (None, np.arange(8, dtype=np.int32) * 7, np.array([5], np.int32)):
        sel = range(B) if rows is None else rows
        say("sampled parity at T=%g, B=%d K=%d V=%d, %d sequences" % (T, B, K, V, len(sel)))
        acc, out, pad = gpu_accept_sample(zt_d, zd_d, d_d, T, seeds, rows=rows, probs=True)
        acc, out, pad = acc.cpu().numpy(), out.cpu().numpy(), pad.cpu().numpy()
        c = compare_sample(res, acc, out, sel)
        say("  " + str(c) + " accepted=%s" % np.bincount(acc[list(sel)], minlength=K + 1).tolist())
        np.testing.assert_allclose(pad[list(sel)], res.probs_at_draft[list(sel)], rtol=0, atol=PROB_ATOL)
