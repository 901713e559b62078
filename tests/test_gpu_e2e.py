"""End-to-end GPU parity: hidden states and LM-head weights in, committed
tokens and accepted lengths out (spec_verify_logits followed by the accept
calls), against the oracle's fp64 logits and decisions on the same seeded
inputs, for the five benchmark workloads.

The oracle never sees a GPU result: it recomputes the logits in fp64 from the
same bf16/fp32 inputs.  Decisions whose margin is below 1e-4 may differ; they
are counted and printed.  The two largest workloads are compared on a sample
of sequences (the oracle's fp64 contraction per sequence is seconds of CPU).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_support import (ParityCounts, compare_greedy, compare_sample, dev, f64, gpu_accept_greedy,
                         gpu_accept_sample, gpu_logits, say)

pytestmark = pytest.mark.gpu


def _oracle_logits(hidden, W, seqs=None):
    B, P, H = hidden.shape
    h = hidden if seqs is None else hidden[torch.as_tensor(seqs, device=hidden.device)]
    z = oracle.lm_head_logits(f64(h).reshape(-1, H), f64(W))
    return z.reshape(-1, P, W.shape[0])


def test_tiny_workload_1000_rounds_both_modes():
    """fp32, B=1, K=4, H=256, V=1000; hidden and draft noise redrawn every
    round; Philox seed = round; each round verified greedily and sampled."""
    wl = synth.WORKLOADS["tiny_b1_k4_h256_v1000"]
    W = synth.weights(wl)
    Wd = W.to(dev())
    cg, cs = ParityCounts(), ParityCounts()
    w64 = f64(W)
    n_acc = []
    for r in range(1000):
        if r % 250 == 0:
            say("tiny workload round %d" % r)
        inp = synth.round_inputs(wl, r, W=W)
        h = inp["hidden"]
        logits = gpu_logits(h.to(dev()), Wd)
        zd, d = inp["draft_logits"], inp["drafts"]
        dg = torch.argmax(zd, dim=-1).to(torch.int32)          # greedy drafts for the greedy pass
        acc_g, out_g = gpu_accept_greedy(logits, dg.to(dev()))
        acc_s, out_s, _ = gpu_accept_sample(logits, zd.to(dev()), d.to(dev()), wl.temperature, inp["seeds"])
        z64 = oracle.lm_head_logits(f64(h).reshape(-1, wl.H), w64).reshape(1, wl.K + 1, wl.V)
        cg.merge(compare_greedy(oracle.accept_greedy(z64, dg.numpy()), acc_g.cpu().numpy(), out_g.cpu().numpy(), [0]))
        rs = oracle.accept_sample(z64, zd.numpy(), d.numpy(), wl.temperature, inp["seeds"])
        cs.merge(compare_sample(rs, acc_s.cpu().numpy(), out_s.cpu().numpy(), [0]))
        n_acc.append(int(acc_s[0]))
    say("tiny greedy: %s" % cg)
    say("tiny sampled: %s  mean accepted %.3f" % (cs, np.mean(n_acc)))
    assert cg.rows == 1000 and cs.rows == 1000


def test_b1_k5_many_seeds():
    """B=1, K=5, H=4096, V=128256, bf16; W, hidden and draft logits fixed;
    drafts redrawn from the draft distribution and seed = round."""
    wl = synth.WORKLOADS["b1_k5_h4096_v128256"]
    say("b1_k5: generating inputs")
    W = synth.weights(wl, dev())
    h = synth.hidden_states(wl, dev())
    base = synth.base_logits(h, W)
    zd = synth.draft_logits(wl, base)
    logits = gpu_logits(h, W)
    z64 = _oracle_logits(h, W)
    zd64 = zd.cpu().numpy()
    c = ParityCounts()
    hist = np.zeros(wl.K + 1, int)
    for r in range(64):
        d = synth.draft_tokens(zd, np.ones(1, bool), wl.temperature, seed=10_000 + r)
        seeds = synth.seeds(wl, r)
        acc, out, _ = gpu_accept_sample(logits, zd, d, wl.temperature, seeds)
        res = oracle.accept_sample(z64, zd64, d.cpu().numpy(), wl.temperature, seeds)
        c.merge(compare_sample(res, acc.cpu().numpy(), out.cpu().numpy(), [0]))
        hist[int(acc[0])] += 1
    say("b1_k5 sampled: %s accepted-length histogram %s" % (c, hist.tolist()))


def _run_mixed(wl, seqs_checked, rnd=0):
    say("%s: generating inputs on the GPU" % wl.name)
    W = synth.weights(wl, dev())
    h = synth.hidden_states(wl, dev(), rnd)
    base = synth.base_logits(h, W)
    zd = synth.draft_logits(wl, base, rnd)
    smask = synth.sampled_mask(wl, rnd)
    d = synth.draft_tokens(zd, smask, wl.temperature, seed=wl.data_seed * 104729 + rnd)
    seeds = synth.seeds(wl, rnd)
    greedy_rows = np.nonzero(~smask)[0]
    sampled_rows = np.nonzero(smask)[0]
    say("%s: GPU verify step (%d greedy, %d sampled rows)" % (wl.name, len(greedy_rows), len(sampled_rows)))
    logits = gpu_logits(h, W)
    acc = torch.full((wl.B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((wl.B, wl.K + 1), -9, dtype=torch.int32, device=dev())
    if len(greedy_rows):
        gpu_accept_greedy(logits, d, rows=greedy_rows, acc=acc, out=out)
    if len(sampled_rows):
        gpu_accept_sample(logits, zd, d, wl.temperature, seeds, rows=sampled_rows, acc=acc, out=out)
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    assert np.all(acc >= 0)
    say("%s: oracle on %d sequences" % (wl.name, len(seqs_checked)))
    seqs = np.asarray(seqs_checked)
    z64 = _oracle_logits(h, W, seqs)
    zd64 = zd[torch.as_tensor(seqs, device=dev())].cpu().numpy()
    dd = d[torch.as_tensor(seqs, device=dev())].cpu().numpy()
    loc_g = [k for k, b in enumerate(seqs) if not smask[b]]
    loc_s = [k for k, b in enumerate(seqs) if smask[b]]
    c = ParityCounts()
    if loc_g:
        rg = oracle.accept_greedy(z64, dd, rows=loc_g)
        c.merge(compare_greedy(rg, acc[seqs], out[seqs], loc_g))
    if loc_s:
        rs = _sample_at_slots(z64, zd64, dd, wl, seeds, seqs, loc_s)
        c.merge(compare_sample(rs, acc[seqs], out[seqs], loc_s))
    say("%s: %s; accepted-length histogram %s" % (wl.name, c, np.bincount(acc, minlength=wl.K + 1).tolist()))


def _sample_at_slots(z64, zd64, dd, wl, seeds, seqs, loc_s):
    """Oracle sampled acceptance of a subset of sequences, each keeping its
    own batch slot b (the Philox counter uses b): embed the subset in a
    batch of B rows where only the checked rows carry data (np.zeros pages
    that are never written cost no memory)."""
    B, P, V = wl.B, wl.K + 1, wl.V
    zt_full = np.zeros((B, P, V))
    zd_full = np.zeros((B, wl.K, V))
    d_full = np.zeros((B, wl.K), np.int64)
    slots = seqs[loc_s]
    zt_full[slots] = z64[loc_s]
    zd_full[slots] = zd64[loc_s]
    d_full[slots] = dd[loc_s]
    res = oracle.accept_sample(zt_full, zd_full, d_full, wl.temperature, seeds, rows=slots)
    # back to the subset's local indexing
    for f in ("accepted_len", "out_tokens", "accept_margin", "terminal_margin"):
        arr = getattr(res, f)
        loc = np.full((len(seqs),) + arr.shape[1:], arr.flat[0], dtype=arr.dtype)
        loc[loc_s] = arr[slots]
        setattr(res, f, loc)
    return res


def test_b64_k4_full_batch():
    wl = synth.WORKLOADS["b64_k4_h4096_v128256"]
    _run_mixed(wl, np.arange(wl.B))


def test_b256_k8_sampled_sequences():
    wl = synth.WORKLOADS["b256_k8_h8192_v152064"]
    _run_mixed(wl, np.array([0, 1, 77, 128, 200, 255]))


def test_b512_k3_sampled_sequences():
    wl = synth.WORKLOADS["b512_k3_h5120_v262144"]
    smask = synth.sampled_mask(wl)
    g = np.nonzero(~smask)[0][:4]
    s = np.nonzero(smask)[0][:4]
    _run_mixed(wl, np.concatenate([g, s, [wl.B - 1]]))
