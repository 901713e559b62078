"""End-to-end GPU parity on the tiny fp32 workload (B=1, K=4, H=256, V=1000):
hidden states and LM-head weights in, committed tokens and accepted lengths
out (spec_verify_logits followed by the accept calls), against the oracle's
fp64 logits and decisions, over its 1000 rounds (hidden states and draft
noise redrawn every round, Philox seed = round), each round verified
greedily and by sampling.

The oracle never sees a GPU result in end-to-end mode: it recomputes the
logits in fp64 from the same fp32 inputs.  A second comparison runs the
oracle on the GPU's fp32 logits (accept only).  Decisions are compared one
by one under the stated 1e-4 rule and the derived rounding bound (see
gpu_support); counts per decision type go to $SV_PARITY_OUT when set.  The
four bf16 workloads are checked in full in test_gpu_parity_full.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_support import (NEAR_TIE, Tally, dev, f64, gpu_accept_greedy, gpu_accept_sample, gpu_logits,
                         sample_bound_ctx, say, strict_greedy, strict_sample, write_counts)

pytestmark = pytest.mark.gpu


def test_tiny_workload_1000_rounds_both_modes():
    wl = synth.WORKLOADS["tiny_b1_k4_h256_v1000"]
    W = synth.weights(wl)
    Wd = W.to(dev())
    w64 = f64(W)
    T = wl.temperature
    te_g, ta_g, te_s, ta_s = Tally(), Tally(), Tally(), Tally()
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
        acc_s, out_s, _ = gpu_accept_sample(logits, zd.to(dev()), d.to(dev()), T, inp["seeds"])
        acc_g, out_g, acc_s, out_s = (x.cpu().numpy() for x in (acc_g, out_g, acc_s, out_s))
        z64 = oracle.lm_head_logits(f64(h).reshape(-1, wl.H), w64).reshape(1, wl.K + 1, wl.V)
        zg = logits.cpu().numpy().astype(np.float64)
        delta = np.max(np.abs(zg - z64), axis=-1)
        zdn, dn = zd.numpy().astype(np.float64), d.numpy()
        strict_greedy(oracle.accept_greedy(z64, dg.numpy()), acc_g, out_g, [0], delta=delta.max(axis=1), tally=te_g)
        strict_greedy(oracle.accept_greedy(zg, dg.numpy()), acc_g, out_g, [0], delta=None, tally=ta_g)
        for z, tally, dl in ((z64, te_s, delta), (zg, ta_s, None)):
            probs = oracle.sample_probs(z, zdn, dn, T)
            res = oracle.accept_sample_probs(probs, dn, inp["seeds"])
            strict_sample(res, acc_s, out_s, [0], sample_bound_ctx(probs, z, zdn, T, delta=dl), dn, tally)
        n_acc.append(int(acc_s[0]))
    te, ta = te_g.merge(te_s), ta_g.merge(ta_s)
    say("tiny end to end:  %s" % te)
    say("tiny accept only: %s" % ta)
    say("tiny sampled: mean accepted %.3f" % np.mean(n_acc))
    assert te.rows == 2000 and ta.rows == 2000
    write_counts("parity_tiny_b1_k4_h256_v1000", dict(
        workload="tiny_b1_k4_h256_v1000", rounds=1000, sequences=1,
        note="each round verified once greedily (drafts = argmax of the draft logits) and once by sampling",
        near_tie_threshold=NEAR_TIE, end_to_end=te.as_dict(), accept_only=ta.as_dict(),
        mean_accepted_sampled=float(np.mean(n_acc)),
        command="SV_PARITY_OUT=<dir> python -m pytest tests/test_gpu_e2e.py -m gpu"))
