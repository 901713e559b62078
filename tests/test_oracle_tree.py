"""Pins of the oracle's greedy tree verification.

  * a chain (every node's parent is the node before it) is a linear draft:
    the result equals the linear greedy rule on the same tokens, itself
    pinned by brute force;
  * brute force against target-only greedy decoding, the property the pages
    fix for greedy verification ("Inference-4", greedy bullet): with a toy
    context-dependent target, every node's logits come from its own path,
    and the committed tokens must be the first d+1 tokens of target-only
    greedy decoding, d the depth of the deepest node whose whole path agrees
    with that decoding -- found here by comparing paths, not by the
    parent-argmax recursion the oracle runs;
  * a star (every node a child of the root) accepts one token exactly when a
    child holds the root's argmax;
  * relabelling the nodes in another topological order changes nothing but
    the node indices;
  * malformed trees and bad rows are faults.
"""
import zlib

import numpy as np
import pytest

import oracle

V, H = 8, 16


class ToyTarget:
    """logits(prefix) = W · h(prefix), h a seeded hash of the token prefix."""

    def __init__(self, seed):
        self.W = np.random.default_rng(seed).normal(size=(V, H))

    def logits(self, prefix):
        key = zlib.crc32(np.asarray(prefix, np.int64).tobytes())
        return self.W @ np.random.default_rng(key).normal(size=H)

    def greedy(self, prefix, n):
        seq = list(prefix)
        for _ in range(n):
            seq.append(int(np.argmax(self.logits(seq))))
        return seq[len(prefix):]


def _random_tree(N, rng, distinct_siblings=True, follow=None):
    """parents[v] < v; tokens random in [0, V) (distinct among siblings if
    asked); with ``follow`` = (target, prefix), tokens copy the target's
    greedy choice with probability 0.6 so deep paths get accepted."""
    par = np.zeros(N + 1, np.int64)
    tok = np.zeros(N + 1, np.int64)
    used = {0: set()}
    paths = {0: []}
    for v in range(1, N + 1):
        par[v] = v - 1 - min(v - 1, rng.geometric(0.45) - 1)
        p = par[v]
        choices = [t for t in range(V) if not (distinct_siblings and t in used[p])]
        if not choices:
            par[v] = p = 0
            choices = [t for t in range(V) if not (distinct_siblings and t in used[0])] or list(range(V))
        t = int(rng.choice(choices))
        if follow is not None and rng.random() < 0.6:
            tgt, prefix = follow
            g = int(np.argmax(tgt.logits(list(prefix) + paths[p])))
            if not distinct_siblings or g not in used[p]:
                t = g
        tok[v] = t
        used[p].add(t)
        used[v] = set()
        paths[v] = paths[p] + [t]
    return par, tok, paths


def test_chain_equals_linear_rule():
    rng = np.random.default_rng(0)
    B, N, Vb = 12, 9, 300
    z = rng.normal(0, 2, (B, N + 1, Vb))
    am = np.argmax(z, axis=-1)
    d = np.where(rng.random((B, N)) < 0.8, am[:, :N], rng.integers(0, Vb, (B, N)))
    par = np.tile(np.arange(-1, N), (B, 1))
    tok = np.concatenate([np.zeros((B, 1), np.int64), d], axis=1)
    t = oracle.tree_accept_greedy(z, par, tok)
    g = oracle.accept_greedy(z, d)
    np.testing.assert_array_equal(t.accepted_len, g.accepted_len)
    np.testing.assert_array_equal(t.out_tokens, g.out_tokens)
    for b in range(B):
        n = g.accepted_len[b]
        assert t.out_nodes[b, :n].tolist() == list(range(1, n + 1)) and np.all(t.out_nodes[b, n:] == -1)


@pytest.mark.parametrize("seed,prefix,N", [(0, [1, 2, 3], 20), (1, [5], 40), (2, [0, 7, 4], 63), (3, [6, 1], 12)])
def test_bruteforce_equals_target_only_greedy(seed, prefix, N):
    tgt = ToyTarget(seed)
    rng = np.random.default_rng(100 + seed)
    B = 16
    ref = tgt.greedy(prefix, N + 1)
    z = np.empty((B, N + 1, V))
    pars, toks, expect = [], [], []
    for b in range(B):
        par, tok, paths = _random_tree(N, rng, distinct_siblings=(b % 2 == 0), follow=(tgt, prefix))
        for v in range(N + 1):
            z[b, v] = tgt.logits(list(prefix) + paths[v])
        # deepest node whose path is a prefix of the greedy decoding (lowest index on ties)
        best = max(range(N + 1), key=lambda v: (paths[v] == ref[:len(paths[v])], len(paths[v]), -v))
        assert paths[best] == ref[:len(paths[best])]
        expect.append((best, len(paths[best])))
        pars.append(par)
        toks.append(tok)
    res = oracle.tree_accept_greedy(z, np.array(pars), np.array(toks))
    depths = []
    for b, (best, d) in enumerate(expect):
        assert res.accepted_len[b] == d
        assert res.out_tokens[b, :d + 1].tolist() == ref[:d + 1]
        assert np.all(res.out_tokens[b, d + 1:] == -1)
        assert res.out_nodes[b, d - 1] == best if d else res.out_nodes[b, 0] == -1
        depths.append(d)
    assert max(depths) >= 2    # the trees do reach past the first level


def test_star_tree():
    rng = np.random.default_rng(5)
    B, N, Vb = 20, 6, 50
    z = rng.normal(0, 1, (B, N + 1, Vb))
    par = np.zeros((B, N + 1), np.int64)
    tok = rng.integers(0, Vb, (B, N + 1))
    a0 = np.argmax(z[:, 0], axis=-1)
    tok[::2, 3] = a0[::2]
    res = oracle.tree_accept_greedy(z, par, tok)
    for b in range(B):
        hit = np.nonzero(tok[b, 1:] == a0[b])[0]
        if len(hit):
            v = hit[0] + 1
            assert res.accepted_len[b] == 1 and res.out_nodes[b, 0] == v
            assert res.out_tokens[b, :2].tolist() == [a0[b], np.argmax(z[b, v])]
        else:
            assert res.accepted_len[b] == 0 and res.out_tokens[b, 0] == a0[b]


def test_relabelling_changes_only_node_indices():
    tgt = ToyTarget(7)
    prefix = [3, 3]
    rng = np.random.default_rng(8)
    N = 30
    par, tok, paths = _random_tree(N, rng, follow=(tgt, prefix))
    z = np.array([tgt.logits(prefix + paths[v]) for v in range(N + 1)])
    # another topological order: BFS order of the same tree
    children = {v: [] for v in range(N + 1)}
    for v in range(1, N + 1):
        children[par[v]].append(v)
    order = [0]
    for v in order:
        order.extend(children[v])
    new_of = {old: new for new, old in enumerate(order)}
    par2 = np.array([0] + [new_of[par[old]] for old in order[1:]])
    tok2 = tok[order]
    a = oracle.tree_accept_greedy(z[None], par[None], tok[None])
    b = oracle.tree_accept_greedy(z[order][None], par2[None], tok2[None])
    assert a.accepted_len[0] == b.accepted_len[0]
    np.testing.assert_array_equal(a.out_tokens, b.out_tokens)
    n = a.accepted_len[0]
    assert [new_of[v] for v in a.out_nodes[0, :n]] == b.out_nodes[0, :n].tolist()


def test_faults():
    rng = np.random.default_rng(9)
    B, N, Vb = 4, 5, 40
    z = rng.normal(0, 1, (B, N + 1, Vb))
    par = np.tile(np.array([0, 0, 1, 1, 2, 0]), (B, 1))
    tok = rng.integers(0, Vb, (B, N + 1))
    par[1, 3] = 3          # not topological
    tok[2, 5] = Vb         # token out of range
    z[3, 4, 7] = np.nan    # bad row
    res = oracle.tree_accept_greedy(z, par, tok)
    assert res.accepted_len.tolist()[1:] == [-1, -1, -1] and res.accepted_len[0] >= 0
    assert np.all(res.out_tokens[1:] == -1)
