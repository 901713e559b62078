"""The one-launch acceptance + residual draw of small sampled batches has two
ways to reach the terminal token once the chunk sums are in, and a bounded
wait in front of one of them:

* at most 256 workgroups: each publishes its chunk sum in a tagged slot and
  polls the others; the owner of the chosen chunk picks the token from its
  registers;
* more: the sums are counted in and the last workgroup selects, re-reading
  the chosen chunk;
* a workgroup whose poll runs out of rounds (forced here with a bound of 0
  from the host) sums every chunk itself and writes the token if it owns the
  chosen chunk.

The residual draw that follows a separate acceptance launch polls the same
way for moderate batches (one slot per 4096-entry chunk, a group of chunks
per workgroup) and counts its blocks in beyond that.

All three evaluate the same weights with the same reductions, so their
tokens must be identical, bit for bit.  Both end-of-draw cases occur in the
rounds below (a
rejection with a residual draw, all drafts accepted with a bonus draw), and
the step at B=1 (cooperative LM head, which zeroes the slots) is covered the
same way.  Oracle parity of these paths is checked by the accept, step and
full-size parity tests; here only their agreement is.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_02_amd as sv
from gpu_support import dev, gpu_accept_sample, say, seeds_tensor

pytestmark = pytest.mark.gpu


def _round(B, K, V, seed, sigma):
    g = torch.Generator().manual_seed(seed)
    zt = torch.randn((B, K + 1, V), generator=g) * 2.0
    zd = zt[:, :K] + torch.randn((B, K, V), generator=g) * sigma
    u = torch.rand((B, K, V), generator=g, dtype=torch.float64).clamp_(min=1e-300)
    d = torch.argmax(zd.double() - torch.log(-torch.log(u)), dim=-1).to(torch.int32)
    return zt, zd, d


def _with_limit(limit, fn):
    prev = sv.spec_set_poll_limit(limit)
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        sv.spec_set_poll_limit(prev)


@pytest.mark.parametrize("V", [5003, 128256])
def test_polled_counted_and_give_up_agree(V):
    B, K, T = 3, 5, 1.0
    kinds = set()
    for rnd in range(6):
        # sigma 0.05: drafts close to the target, so some rounds accept all
        zt, zd, d = _round(B, K, V, seed=1000 * rnd + V % 977, sigma=0.05 if rnd % 2 else 1.5)
        zt, zd, d = zt.to(dev()), zd.to(dev()), d.to(dev())
        seeds = np.arange(B, dtype=np.uint64) * 104729 + rnd
        say("poll paths V=%d round %d" % (V, rnd))
        polled = _with_limit(-1, lambda: gpu_accept_sample(zt, zd, d, T, seeds, rows=[0, 1], probs=True))
        gave_up = _with_limit(0, lambda: gpu_accept_sample(zt, zd, d, T, seeds, rows=[0, 1], probs=True))
        wider = _with_limit(-1, lambda: gpu_accept_sample(zt, zd, d, T, seeds, rows=[0, 1, 2], probs=True))
        every = _with_limit(-1, lambda: gpu_accept_sample(zt, zd, d, T, seeds, probs=True))
        p_acc, p_out, p_pad = (x.cpu().numpy() for x in polled)
        for other in (gave_up, wider, every):
            o_acc, o_out, o_pad = (x.cpu().numpy() for x in other)
            np.testing.assert_array_equal(p_acc[:2], o_acc[:2])
            np.testing.assert_array_equal(p_out[:2], o_out[:2])
            np.testing.assert_array_equal(p_pad[:2], o_pad[:2])
        for b in range(2):
            n = int(p_acc[b])
            assert 0 <= n <= K
            assert 0 <= p_out[b, n] < V
            kinds.add("bonus" if n == K else "residual")
    assert kinds == {"bonus", "residual"}, kinds


def test_step_b1_poll_give_up_agrees():
    """spec_verify_step at B=1 (cooperative LM head with the statistics; it
    zeroes the poll slots), default bound against a bound of 0."""
    B, K, H, V, T = 1, 5, 512, 128256, 1.0
    g = torch.Generator().manual_seed(5)
    hidden = torch.randn((B, K + 1, H), generator=g).to(torch.bfloat16).to(dev())
    W = (torch.randn((V, H), generator=g) * 0.05).to(torch.bfloat16).to(dev())
    ws = torch.empty(sv.spec_verify_step_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev())
    kinds = set()
    for rnd in range(8):
        zd = torch.empty((B, K, V), dtype=torch.float32, device=dev())
        logits0 = torch.empty((B, K + 1, V), dtype=torch.float32, device=dev())
        sv.spec_verify_logits(hidden, W, logits0)
        sigma = 0.02 if rnd % 2 else 1.0
        zd.copy_(logits0[:, :K] + sigma * torch.randn((B, K, V), generator=g).to(dev()))
        u = torch.rand((B, K, V), generator=g, dtype=torch.float64).clamp_(min=1e-300).to(dev())
        d = torch.argmax(zd.double() / T - torch.log(-torch.log(u)), dim=-1).to(torch.int32)
        seeds = seeds_tensor(np.array([rnd * 31 + 7], np.uint64))
        res = []
        for limit in (-1, 0):
            logits = torch.full((B, K + 1, V), float("nan"), dtype=torch.float32, device=dev())
            acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
            out = torch.full((B, K + 1), -9, dtype=torch.int32, device=dev())
            pad = torch.full((B, K, 2), float("nan"), dtype=torch.float32, device=dev())
            _with_limit(limit, lambda: sv.spec_verify_step(hidden, W, logits, acc, out, ws, draft_logits=zd,
                                                           draft_tokens=d, temperature=T, seeds=seeds,
                                                           sampled_rows="all", probs_at_draft=pad))
            res.append((logits.cpu(), acc.cpu().numpy(), out.cpu().numpy(), pad.cpu().numpy()))
        say("step B=1 poll bound round %d: accepted %d" % (rnd, int(res[0][1][0])))
        assert torch.equal(res[0][0], res[1][0])
        for a, b in zip(res[0][1:], res[1][1:]):
            np.testing.assert_array_equal(a, b)
        n = int(res[0][1][0])
        assert 0 <= n <= K and 0 <= res[0][2][0, n] < V
        kinds.add("bonus" if n == K else "residual")
    assert kinds == {"bonus", "residual"}, kinds


def test_grouped_polled_residual_matches_counted():
    """The residual draw of moderate batches (acceptance in its own launch):
    at most 256 workgroups sum a group of consecutive 4096-entry chunks each
    and poll one tagged slot per chunk; more sequences than the slots hold
    take the counted path.  32 sequences at V = 128256 (1024 slots, four
    chunks per workgroup) against the same 32 within 65 (counted), and
    against a poll bound of 0; bit for bit."""
    B, K, V, T = 65, 4, 128256, 0.8
    zt, zd, d = _round(B, K, V, seed=4242, sigma=0.3)
    zt, zd, d = zt.to(dev()), zd.to(dev()), d.to(dev())
    kinds = set()
    for rnd in range(3):
        seeds = np.arange(B, dtype=np.uint64) * 7907 + 11 * rnd
        rows32 = list(range(32))
        say("grouped polled residual, round %d" % rnd)
        polled = _with_limit(-1, lambda: gpu_accept_sample(zt, zd, d, T, seeds, rows=rows32, probs=True))
        gave_up = _with_limit(0, lambda: gpu_accept_sample(zt, zd, d, T, seeds, rows=rows32, probs=True))
        counted = _with_limit(-1, lambda: gpu_accept_sample(zt, zd, d, T, seeds, probs=True))
        p_acc, p_out, p_pad = (x.cpu().numpy() for x in polled)
        for other in (gave_up, counted):
            o_acc, o_out, o_pad = (x.cpu().numpy() for x in other)
            np.testing.assert_array_equal(p_acc[:32], o_acc[:32])
            np.testing.assert_array_equal(p_out[:32], o_out[:32])
            np.testing.assert_array_equal(p_pad[:32], o_pad[:32])
        for b in range(32):
            n = int(p_acc[b])
            assert 0 <= n <= K and 0 <= p_out[b, n] < V
            kinds.add("bonus" if n == K else "residual")
    assert kinds == {"bonus", "residual"}, kinds
