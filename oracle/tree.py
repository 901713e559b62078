"""fp64 CPU definition of greedy verification of a draft tree.

A tree drafter proposes several candidate continuations at once: each node
holds one candidate token and hangs under the node whose continuation it
extends; the target scores every node in one forward pass, each node seeing
only the root and its own ancestors, and the longest path the target agrees
with is kept ("Inference-4", Medusa; "speculative-decoding" blog, Medusa and
EAGLE-2's dynamic draft trees; "Speculative decoding" course page, One pass,
many candidate continuations).  The greedy rule is the linear rule applied
along every root-to-node path:

  node 0 is the root (the last accepted token); node v >= 1 has parent
  p(v) < v and token d_v; a_u = argmax_v' logits[u, v'] (lowest index on ties)
  is the target's next token after the path to u.
  accepted(0) = true;  accepted(v) = accepted(p(v)) and d_v == a_{p(v)}.
  The kept node is the accepted node of greatest depth (lowest index among
  equals); its path root -> node gives the committed drafts, and a at the kept
  node is the bonus token.

Readings where the pages are silent: ties between equally deep accepted
nodes (possible only when siblings repeat a token) go to the lowest node
index; a sequence whose parents are not in topological order (p(v) outside
[0, v)) or whose tokens fall outside [0, V) is a data fault, as is a NaN or
+inf logit, or a node row with no finite entry, anywhere in its tree.

Part of the oracle (test infrastructure); see oracle/__init__.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .verify import _bad_rows, _rows_arg, _top2_margin


@dataclass
class TreeResult:
    accepted_len: np.ndarray   # [B] int32: depth of the kept node; -1 fault, -2 not selected
    out_tokens: np.ndarray     # [B, N+1] int32: path tokens, bonus token, then -1
    out_nodes: np.ndarray      # [B, N+1] int32: node index of each committed draft, then -1
    argmax: np.ndarray         # [B, N+1] target argmax per node
    margin: np.ndarray         # [B, N+1] top1 - top2 per node row


def tree_accept_greedy(logits, parents, tokens, rows=None) -> TreeResult:
    """logits [B, N+1, V] (row v = the target's logits after the path to node
    v); parents, tokens [B, N+1] int (entry 0, the root, is ignored)."""
    z = np.asarray(logits, dtype=np.float64)
    par = np.asarray(parents, dtype=np.int64)
    tok = np.asarray(tokens, dtype=np.int64)
    B, P, V = z.shape
    N = P - 1
    acc = np.full(B, -2, np.int32)
    out = np.full((B, P), -1, np.int32)
    nodes = np.full((B, P), -1, np.int32)
    amax = np.full((B, P), -1, np.int64)
    marg = np.full((B, P), np.inf)
    for b in _rows_arg(rows, B):
        v = np.arange(1, P)
        if (np.any(_bad_rows(z[b])) or np.any((par[b, 1:] < 0) | (par[b, 1:] >= v))
                or np.any((tok[b, 1:] < 0) | (tok[b, 1:] >= V))):
            acc[b] = -1
            continue
        a = np.argmax(z[b], axis=-1)
        amax[b] = a
        marg[b] = _top2_margin(z[b])
        ok = np.zeros(P, bool)
        depth = np.zeros(P, np.int64)
        ok[0] = True
        best = 0
        for u in range(1, P):
            p = par[b, u]
            depth[u] = depth[p] + 1
            ok[u] = ok[p] and tok[b, u] == a[p]
            if ok[u] and depth[u] > depth[best]:
                best = u
        path = []
        u = best
        while u != 0:
            path.append(u)
            u = par[b, u]
        path.reverse()
        n = len(path)
        out[b, :n] = tok[b, path]
        out[b, n] = a[best]
        nodes[b, :n] = path
        acc[b] = n
    return TreeResult(acc, out, nodes, amax, marg)
