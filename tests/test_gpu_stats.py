"""Statistical checks of the GPU sampled path against what the pages fix.

* The committed tokens are distributed as the target: chi-square over 10^6
  verify rounds of the GPU kernels (fixed logits, drafts redrawn from the
  draft distribution each round, one Philox seed per round), per position,
  against softmax(z/T) computed by scipy ("Inference-4", sampling bullet;
  "speculative-decoding" blog, Rejection sampling).
* Mean tokens per round = (1 - a^(K+1)) / (1 - a) for constructed pairs with
  constant acceptance probability a ("Inference-4", The idea; "What is
  speculative decoding" guide, its worked example at gamma = 4, a = 0.7).
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

from gpu_support import dev, gpu_accept_sample, say

pytestmark = pytest.mark.gpu


def _chisq_p(tokens, probs):
    V = len(probs)
    obs = np.bincount(tokens, minlength=V).astype(np.float64)
    exp = probs * obs.sum()
    small = exp < 5
    o = np.append(obs[~small], obs[small].sum())
    e = np.append(exp[~small], exp[small].sum())
    keep = e > 0
    assert np.all(o[~keep] == 0), "a token with zero target probability was emitted"
    return stats.chisquare(o[keep], e[keep] * o[keep].sum() / e[keep].sum()).pvalue


def _rounds(zt, zd, T, n_rounds, per_call=10_000, seed0=0):
    """n_rounds verify rounds on the GPU: B = per_call sequences per call, all
    with the same logits; sequence b of call k uses seed seed0 + k*per_call + b."""
    P, V = zt.shape
    K = P - 1
    ztd = zt.to(dev()).expand(per_call, P, V).contiguous()
    zdd = zd.to(dev()).expand(per_call, K, V).contiguous()
    pd = torch.softmax(zd.double().to(dev()) / T, dim=-1)
    g = torch.Generator(device=dev())
    g.manual_seed(1234)
    accs, toks = [], []
    for k in range(n_rounds // per_call):
        d = torch.stack([torch.multinomial(pd[i], per_call, replacement=True, generator=g) for i in range(K)],
                        dim=-1).to(torch.int32)
        seeds = np.arange(seed0 + k * per_call, seed0 + (k + 1) * per_call, dtype=np.uint64)
        acc, out, _ = gpu_accept_sample(ztd, zdd, d, T, seeds)
        accs.append(acc.cpu().numpy())
        toks.append(out.cpu().numpy())
    return np.concatenate(accs), np.concatenate(toks)


@pytest.mark.parametrize("V,K,T", [(1000, 4, 1.0), (64, 3, 0.7)])
def test_chisquare_1e6_rounds(V, K, T):
    say("chi-square: 1e6 GPU rounds V=%d K=%d T=%g" % (V, K, T))
    g = torch.Generator().manual_seed(V + K)
    zt = torch.randn((K + 1, V), generator=g) * 1.5
    zd = zt[:K] + torch.randn((K, V), generator=g)
    acc, tok = _rounds(zt, zd, T, 1_000_000)
    q = special.softmax(zt.double().numpy() / T, axis=-1)
    pv = []
    for i in range(K + 1):
        reached = acc >= i
        pv.append(_chisq_p(tok[reached, i], q[i]))
    say("  p-values per position %s; accepted-length histogram %s"
        % (["%.3g" % p for p in pv], np.bincount(acc, minlength=K + 1).tolist()))
    assert min(pv) > 1e-3


@pytest.mark.parametrize("alpha", [0.0, 0.7, 1.0])
def test_expected_tokens_constant_alpha(alpha):
    """Target q on tokens 0..V-2 plus a sink token whose target logit is -1e4
    (probability 0 in fp32 too); draft p = alpha*q on the support, 1-alpha on
    the sink: each draft is accepted with probability exactly alpha."""
    K, V, N = 4, 16, 200_000
    g = torch.Generator().manual_seed(int(alpha * 100))
    zts, zds = [], []
    for _ in range(K + 1):
        zt = torch.cat([torch.randn(V - 1, generator=g, dtype=torch.float64), torch.tensor([-1e4], dtype=torch.float64)])
        q = torch.softmax(zt, 0)
        p = torch.cat([alpha * q[:-1], torch.tensor([1.0 - alpha], dtype=torch.float64)])
        zts.append(zt)
        zds.append(torch.log(p))
    zt = torch.stack(zts).float()
    zd = torch.stack(zds[:K]).float()
    acc, _ = _rounds(zt, zd, 1.0, N, per_call=20_000, seed0=int(alpha * 1e8))
    tokens = acc + 1.0
    expect = K + 1.0 if alpha == 1.0 else (1 - alpha ** (K + 1)) / (1 - alpha)
    se = tokens.std(ddof=1) / np.sqrt(N)
    say("alpha=%g: mean tokens %.4f, closed form %.4f, se %.4f" % (alpha, tokens.mean(), expect, se))
    assert abs(tokens.mean() - expect) <= 4 * se + 1e-9
