"""fp64 CPU definition of the speculative-decoding verify step.

Notation: q = target distribution, p = draft distribution ("Inference-4"
names them the other way round; the other pages, and this code, call the
target's distribution the one in the numerator of the accept ratio).  Every
function below is written from the pages' description, in their order:

  1. LM-head logits of the K+1 verify positions (the target runs one pass over
     the last accepted token and the K drafts and yields K+1 distributions:
     "Inference-4", Draft-model speculative decoding, step 2).
  2. Greedy acceptance: accept drafts while they equal the target's most
     likely token; at the first mismatch emit the target's token; if all K
     match, emit the bonus token from the position after the last draft
     (same page, greedy bullet, and its generate_speculative listing).
  3. Speculative sampling: accept draft x with probability min(1, q(x)/p(x)),
     left to right, stop at the first rejection and draw the replacement from
     norm(max(0, q - p)); if every draft is accepted, draw the bonus token from
     the target's distribution after the last draft ("Inference-4", sampling
     bullet; "speculative-decoding" blog, Rejection sampling section;
     "Speculative decoding" course page, Why this is not approximate; "What is
     speculative decoding" guide, How speculative decoding works).

Readings where the pages are silent (each is listed in the design notes):
ties in argmax go to the lowest index; temperature T divides target and
draft logits alike; the accept test is u < r with u on a 24-bit grid from
Philox word 0 and the terminal draw uses Philox word 1; the terminal draw is
an inverse CDF over the in-order cumulative sum of the weights; if the
residual mass is zero the draw falls back to q.

Rows with bad data (a draft token outside [0, V), a NaN or +inf logit, or a
row whose maximum is -inf) are marked: accepted_len = -1, out_tokens all -1.

Part of the oracle (test infrastructure); see oracle/__init__.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import verify_uniforms


# ---------------------------------------------------------------- inputs ----

def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------- step 1: logits --

def lm_head_logits(hidden, W, chunk: int = 4096) -> np.ndarray:
    """logits[m, v] = sum_h hidden[m, h] * W[v, h], accumulated in fp64.

    hidden: [M, H]; W: [V, H] (any float dtype; bf16 inputs are widened with
    ``widen_bf16`` first).  The products of bf16 or fp32 inputs are exact in
    fp64; only the summation rounds.  Chunked over V to bound memory.
    """
    x = np.asarray(hidden, dtype=np.float64)
    M, H = x.shape
    V = W.shape[0]
    out = np.empty((M, V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        out[:, v0:v1] = x @ np.asarray(W[v0:v1], dtype=np.float64).T
    return out


# ------------------------------------------------------------ helpers ------

def softmax(z, T: float) -> np.ndarray:
    """softmax(z / T) along the last axis, shifted by the row maximum."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp((z - m) / T)
    return e / np.sum(e, axis=-1, keepdims=True)


def _bad_rows(z) -> np.ndarray:
    """True for rows (last axis) holding NaN or +inf, or whose max is -inf."""
    z = np.asarray(z)
    if z.shape[-1] == 0:
        return np.ones(z.shape[:-1], bool)
    nan_or_pinf = np.any(np.isnan(z) | (z == np.inf), axis=-1)
    all_ninf = np.all(z == -np.inf, axis=-1)
    return nan_or_pinf | all_ninf


def _top2_margin(z) -> np.ndarray:
    """top1 - top2 of each row (inf when the row has one entry)."""
    z = np.asarray(z, dtype=np.float64)
    if z.shape[-1] < 2:
        return np.full(z.shape[:-1], np.inf)
    part = -np.partition(-z, 1, axis=-1)[..., :2]
    return part[..., 0] - part[..., 1]


def _rows_arg(rows, B):
    if rows is None:
        return np.arange(B)
    return np.asarray(rows, dtype=np.int64)


# ------------------------------------------------ step 2: greedy accept ----

@dataclass
class GreedyResult:
    accepted_len: np.ndarray      # [B] int32: n (0..K), -1 bad row, -2 row not selected
    out_tokens: np.ndarray        # [B, K+1] int32, -1 past the emitted token
    argmax: np.ndarray            # [B, K+1] target argmax per position
    margin: np.ndarray            # [B, K+1] top1 - top2 of the target logits


def accept_greedy(logits, draft_tokens, rows=None) -> GreedyResult:
    """Greedy verification of each selected row b.

    a_i = argmax_v logits[b, i, v] (lowest index on ties), i = 0..K.
    n = number of leading drafts with d_i == a_i.  Emitted: d_0..d_{n-1}, a_n.
    """
    z = np.asarray(logits, dtype=np.float64)
    d = np.asarray(draft_tokens, dtype=np.int64)
    B, P, V = z.shape
    K = P - 1
    rows = _rows_arg(rows, B)
    acc = np.full(B, -2, np.int32)
    out = np.full((B, K + 1), -1, np.int32)
    amax = np.full((B, K + 1), -1, np.int64)
    marg = np.full((B, K + 1), np.inf)
    for b in rows:
        bad = bool(np.any(_bad_rows(z[b])))
        if K and np.any((d[b] < 0) | (d[b] >= V)):
            bad = True
        if bad:
            acc[b] = -1
            continue
        a = np.argmax(z[b], axis=-1)          # numpy: first maximal index
        amax[b] = a
        marg[b] = _top2_margin(z[b])
        n = 0
        while n < K and d[b, n] == a[n]:
            n += 1
        out[b, :n] = d[b, :n]
        out[b, n] = a[n]
        acc[b] = n
    return GreedyResult(acc, out, amax, marg)


# ------------------------------------------- step 3: speculative sampling ----

@dataclass
class SampleResult:
    accepted_len: np.ndarray      # [B] int32 (-1 bad row, -2 not selected)
    out_tokens: np.ndarray        # [B, K+1] int32
    probs_at_draft: np.ndarray    # [B, K, 2]: q_i(d_i), p_i(d_i)
    ratio: np.ndarray             # [B, K]: r_i = min(1, q_i(d_i)/p_i(d_i))
    u_accept: np.ndarray          # [B, K+1]: Philox word 0 uniforms
    u_terminal: np.ndarray        # [B, K+1]: Philox word 1 uniforms
    accept_margin: np.ndarray     # [B, K]: |u_i - r_i|
    terminal_margin: np.ndarray   # [B]: distance of u'Z to the nearest CDF step, / Z
    residual_mass: np.ndarray     # [B]: Z (sum of the terminal weights)
    alpha: np.ndarray             # [B, K]: sum_v min(q_i, p_i), exact accept prob.


def accept_ratio(q_d, p_d):
    """r = min(1, q/p), with r = 0 where q = 0 and r = 1 where p = 0 < q."""
    q_d = np.asarray(q_d, dtype=np.float64)
    p_d = np.asarray(p_d, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(q_d >= p_d, 1.0, q_d / np.where(p_d > 0, p_d, 1.0))
    return np.where(q_d > 0, np.minimum(r, 1.0), 0.0)


def inverse_cdf(w, u):
    """Inverse-CDF draw over the last axis of w with uniform(s) u.

    t = min{v : C_v > u * Z}, C the in-order cumulative sum of w and
    Z = C_{V-1}.  Returns (t, Z, margin) with margin = min(uZ - C_{t-1},
    C_t - uZ) / Z, the relative distance of the draw point to the nearest
    step of the CDF.  Works on w [..., V] and u [...].
    """
    C = np.cumsum(np.asarray(w, dtype=np.float64), axis=-1)
    V = C.shape[-1]
    Z = C[..., -1]
    x = np.asarray(u, dtype=np.float64) * Z
    t = np.minimum(np.sum(C <= x[..., None], axis=-1), V - 1)   # first C_v > x
    hi = np.take_along_axis(C, t[..., None], axis=-1)[..., 0]
    lo = np.take_along_axis(C, np.maximum(t - 1, 0)[..., None], axis=-1)[..., 0]
    lo = np.where(t > 0, lo, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        margin = np.where(Z > 0, np.minimum(x - lo, hi - x) / Z, 0.0)
    return t, Z, margin


def terminal_weights(q_n, p_n=None):
    """Weights of the terminal draw: max(0, q_n - p_n) after a rejection at n
    (falling back to q_n when that residual has no mass), or q_n itself for
    the bonus position (p_n is None).  Works on [..., V] arrays."""
    q_n = np.asarray(q_n, dtype=np.float64)
    if p_n is None:
        return q_n
    w = np.maximum(0.0, q_n - np.asarray(p_n, dtype=np.float64))
    empty = ~(np.sum(w, axis=-1, keepdims=True) > 0)
    return np.where(empty, q_n, w)


def accept_sample(logits, draft_logits, draft_tokens, temperature, seeds, rows=None, slots=None) -> SampleResult:
    """Speculative sampling of each selected row b (B rows, K drafts, V tokens).

    q_i = softmax(logits[b, i] / T), i = 0..K;  p_i = softmax(draft_logits[b, i] / T), i < K.
    (u_i, u'_i) = Philox uniforms at (seed_b, slot_b, i); slot_b = b unless
    ``slots`` names each row's batch slot.
    Accept d_i iff u_i < r_i = min(1, q_i(d_i)/p_i(d_i)); n = first rejected i, else K.
    Terminal weights: w = max(0, q_n - p_n) if n < K, else q_K (bonus).
    Terminal token: inverse CDF of w at u'_n.  Emitted: d_0..d_{n-1}, t.
    The two halves are ``sample_probs`` (the distributions) and
    ``accept_sample_probs`` (the decisions), for callers that verify many
    rounds over the same logits.
    """
    z = np.asarray(logits)
    B, P, V = z.shape
    rows = _rows_arg(rows, B)
    probs = sample_probs(logits, draft_logits, draft_tokens, temperature, rows)
    return accept_sample_probs(probs, draft_tokens, seeds, slots)


@dataclass
class SampleProbs:
    """The distributions of the selected, well-formed rows of a sampled
    batch: q [R, K+1, V] and p [R, K, V] for the rows ``good`` (in order),
    and alpha [R, K] = sum_v min(q_i, p_i), the probability that a draft
    drawn from p_i is accepted; ``bad`` lists the selected rows marked as
    faulted."""
    B: int
    K: int
    V: int
    good: np.ndarray
    bad: np.ndarray
    q: np.ndarray
    p: np.ndarray
    alpha: np.ndarray


def sample_probs(logits, draft_logits, draft_tokens, temperature, rows=None) -> SampleProbs:
    """q_i = softmax(logits[b, i] / T) and p_i = softmax(draft_logits[b, i] / T)
    of the selected rows; rows with bad data (NaN or +inf, a row without a
    finite entry, a draft token outside [0, V)) are set apart as faulted."""
    z = np.asarray(logits, dtype=np.float64)
    B, P, V = z.shape
    K = P - 1
    zd = np.asarray(draft_logits, dtype=np.float64) if K else np.zeros((B, 0, V))
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(B, K)
    T = float(temperature)
    rows = _rows_arg(rows, B)
    if len(rows) == 0:
        e = np.zeros(0, np.int64)
        return SampleProbs(B, K, V, e, e, np.zeros((0, P, V)), np.zeros((0, K, V)), np.zeros((0, K)))
    zr, zdr, dr = z[rows], zd[rows], d[rows]
    bad = np.any(_bad_rows(zr), axis=-1)
    if K:
        bad |= np.any(_bad_rows(zdr), axis=-1)
        bad |= np.any((dr < 0) | (dr >= V), axis=-1)
    good = rows[~bad]
    q = softmax(z[good], T) if len(good) else np.zeros((0, P, V))
    p = softmax(zd[good], T) if (K and len(good)) else np.zeros((len(good), K, V))
    alpha = np.sum(np.minimum(q[:, :K], p), axis=-1)
    return SampleProbs(B, K, V, good, rows[bad], q, p, alpha)


def accept_sample_probs(probs: SampleProbs, draft_tokens, seeds, slots=None) -> SampleResult:
    """The sampled decisions of the rows in ``probs`` for one round of draft
    tokens [B, K] and seeds [B] (see accept_sample)."""
    B, K, V = probs.B, probs.K, probs.V
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(B, K)
    seeds = np.asarray(seeds, dtype=np.uint64).reshape(B)
    slot = np.arange(B) if slots is None else np.asarray(slots, dtype=np.int64).reshape(B)

    acc = np.full(B, -2, np.int32)
    out = np.full((B, K + 1), -1, np.int32)
    pad = np.full((B, K, 2), np.nan)
    ratio = np.full((B, K), np.nan)
    ua = np.full((B, K + 1), np.nan)
    ut = np.full((B, K + 1), np.nan)
    am = np.full((B, K), np.inf)
    tm = np.full(B, np.inf)
    zz = np.full(B, np.nan)
    alpha = np.full((B, K), np.nan)
    acc[probs.bad] = -1
    good = probs.good
    if len(good) == 0:
        return SampleResult(acc, out, pad, ratio, ua, ut, am, tm, zz, alpha)
    R = len(good)
    q, p, dr = probs.q, probs.p, d[good]
    u, u2 = verify_uniforms(seeds[good][:, None], slot[good][:, None], np.arange(K + 1)[None, :])
    ua[good], ut[good] = u, u2

    ri = np.arange(R)[:, None]
    ki = np.arange(K)[None, :]
    q_d = q[ri, ki, dr]                                  # q_i(d_i)   [R, K]
    p_d = p[ri, ki, dr]                                  # p_i(d_i)
    r = accept_ratio(q_d, p_d)
    pad[good] = np.stack([q_d, p_d], axis=-1)
    ratio[good] = r
    alpha[good] = probs.alpha
    am[good] = np.abs(u[:, :K] - r)

    # n = index of the first rejection (u_i >= r_i), scanning left to right; K if none
    rejected = ~(u[:, :K] < r)
    n = np.where(rejected.any(axis=-1), np.argmax(rejected, axis=-1), K) if K else np.zeros(R, np.int64)

    q_n = q[np.arange(R), n]                             # [R, V]
    w = q_n.copy()
    rej = n < K
    if np.any(rej):
        w[rej] = terminal_weights(q_n[rej], p[np.arange(R)[rej], n[rej]])

    # terminal token: inverse CDF of w at u'_n
    t, Z, margin = inverse_cdf(w, u2[np.arange(R), n])

    for j, b in enumerate(good):
        out[b, :n[j]] = dr[j, :n[j]]
    out[good, n] = t
    acc[good] = n
    tm[good] = margin
    zz[good] = Z
    return SampleResult(acc, out, pad, ratio, ua, ut, am, tm, zz, alpha)


def accept_sample_rounds(probs: SampleProbs, draft_tokens, seeds, slots=None) -> SampleResult:
    """accept_sample_probs over R rounds of the same distributions, with
    draft_tokens [R, B, K] and seeds [R, B]; every result field gains a
    leading round axis.

    Only the draft tokens and the uniforms change from round to round, so
    the terminal weights of each (row, terminal position) and their in-order
    cumulative sums C are formed once; each round then finds its draw in
    them by the same rule, t = min{v : C_v > u' Z} (C is nondecreasing, so
    that is the number of entries C_v <= u' Z), with the same margin.
    """
    B, K, V = probs.B, probs.K, probs.V
    sd = np.asarray(seeds, dtype=np.uint64).reshape(-1, B)
    R = sd.shape[0]
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(R, B, K)
    slot = np.arange(B) if slots is None else np.asarray(slots, dtype=np.int64).reshape(B)
    good = probs.good
    G = len(good)
    q, p = probs.q, probs.p

    # C[j, n]: cumulative terminal weights of good row j when the first
    # rejection is at n (n = K: the bonus draw from q_K)
    C = np.empty((G, K + 1, V))
    for j in range(G):
        for n in range(K + 1):
            w = q[j, n] if n == K else terminal_weights(q[j, n], p[j, n])
            np.cumsum(w, out=C[j, n])
    Ztab = C[:, :, -1]

    acc = np.full((R, B), -2, np.int32)
    out = np.full((R, B, K + 1), -1, np.int32)
    pad = np.full((R, B, K, 2), np.nan)
    ratio = np.full((R, B, K), np.nan)
    ua = np.full((R, B, K + 1), np.nan)
    ut = np.full((R, B, K + 1), np.nan)
    am = np.full((R, B, K), np.inf)
    tm = np.full((R, B), np.inf)
    zz = np.full((R, B), np.nan)
    alpha = np.full((R, B, K), np.nan)
    acc[:, probs.bad] = -1
    if G == 0:
        return SampleResult(acc, out, pad, ratio, ua, ut, am, tm, zz, alpha)
    gi = np.arange(G)[:, None]
    ki = np.arange(K)[None, :]
    for r in range(R):
        dr = d[r, good]
        u, u2 = verify_uniforms(sd[r, good][:, None], slot[good][:, None], np.arange(K + 1)[None, :])
        q_d = q[gi, ki, dr]
        p_d = p[gi, ki, dr]
        rr = accept_ratio(q_d, p_d)
        rejected = ~(u[:, :K] < rr)
        n = np.where(rejected.any(axis=-1), np.argmax(rejected, axis=-1), K) if K else np.zeros(G, np.int64)
        Z = Ztab[np.arange(G), n]
        x = u2[np.arange(G), n] * Z
        t = np.empty(G, np.int64)
        marg = np.empty(G)
        for j in range(G):
            Cj = C[j, n[j]]
            tj = min(int(np.searchsorted(Cj, x[j], side="right")), V - 1)
            lo = Cj[tj - 1] if tj > 0 else 0.0
            t[j] = tj
            marg[j] = min(x[j] - lo, Cj[tj] - x[j]) / Z[j] if Z[j] > 0 else 0.0
        for j, b in enumerate(good):
            out[r, b, :n[j]] = dr[j, :n[j]]
        out[r, good, n] = t
        acc[r, good] = n
        ua[r, good], ut[r, good] = u, u2
        pad[r, good] = np.stack([q_d, p_d], axis=-1)
        ratio[r, good] = rr
        am[r, good] = np.abs(u[:, :K] - rr)
        tm[r, good] = marg
        zz[r, good] = Z
        alpha[r, good] = probs.alpha
    return SampleResult(acc, out, pad, ratio, ua, ut, am, tm, zz, alpha)


# ------------------------------------------- per-sequence draft counts ----
# A drafter may hand back fewer drafts than asked, or none ("Inference-4",
# Prompt lookup decoding, and the draft count its verification loop caps at
# the context window), and a scheduler may pick the count per request
# ("speculative-decoding" blog, DSpark).  Each sequence is then verified on its
# own, exactly as above with K = K_b.  Rows are packed in sequence order:
# sequence b owns target rows row_start[b] .. row_start[b] + K_b and draft
# rows row_start[b] - b .. row_start[b] - b + K_b - 1.

def ragged_sequences(row_start, total_rows: int, K_max: int):
    """(t0, K_b, well_formed) per sequence.  A sequence is well formed when
    0 <= K_b <= K_max, its draft rows start at or after row 0, and its last
    row leaves one row for each later sequence (the entry points' rule)."""
    rs = np.asarray(row_start, dtype=np.int64).reshape(-1)
    B = len(rs) - 1
    out = []
    for b in range(B):
        s0, s1 = int(rs[b]), int(rs[b + 1])
        kb = s1 - s0 - 1
        ok = 0 <= kb <= K_max and s0 >= b and s1 <= total_rows - (B - 1 - b)
        out.append((s0, kb, ok))
    return out


def accept_greedy_ragged(logits, draft_tokens, row_start, K_max: int, rows=None) -> GreedyResult:
    """Greedy verification of a packed batch.  logits [R, V]; draft_tokens
    [R - B].  Result fields are packed: accepted_len [B] (-1 bad or malformed,
    -2 not selected), out_tokens / argmax / margin [R]."""
    z = np.asarray(logits, dtype=np.float64)
    R, V = z.shape
    d = np.asarray(draft_tokens if draft_tokens is not None else np.zeros(0), dtype=np.int64).reshape(-1)
    seqs = ragged_sequences(row_start, R, K_max)
    B = len(seqs)
    acc = np.full(B, -2, np.int32)
    out = np.full(R, -1, np.int32)
    amax = np.full(R, -1, np.int64)
    marg = np.full(R, np.inf)
    for b in _rows_arg(rows, B):
        t0, kb, ok = seqs[b]
        if not ok:
            acc[b] = -1
            continue
        g = accept_greedy(z[None, t0:t0 + kb + 1], d[None, t0 - b:t0 - b + kb])
        acc[b] = g.accepted_len[0]
        out[t0:t0 + kb + 1] = g.out_tokens[0]
        amax[t0:t0 + kb + 1] = g.argmax[0]
        marg[t0:t0 + kb + 1] = g.margin[0]
    return GreedyResult(acc, out, amax, marg)


def accept_sample_ragged(logits, draft_logits, draft_tokens, row_start, K_max: int, temperature, seeds,
                         rows=None) -> SampleResult:
    """Speculative sampling of a packed batch, each sequence in its own batch
    slot b (Philox counter (i, b)).  logits [R, V]; draft_logits [R - B, V];
    draft_tokens [R - B].  Result fields are packed: accepted_len,
    terminal_margin, residual_mass [B]; out_tokens, u_accept, u_terminal [R];
    probs_at_draft [R - B, 2]; ratio, accept_margin, alpha [R - B]."""
    z = np.asarray(logits, dtype=np.float64)
    R, V = z.shape
    seqs = ragged_sequences(row_start, R, K_max)
    B = len(seqs)
    zd = np.asarray(draft_logits, dtype=np.float64) if R > B else np.zeros((0, V))
    d = np.asarray(draft_tokens if draft_tokens is not None else np.zeros(0), dtype=np.int64).reshape(-1)
    seeds = np.asarray(seeds, dtype=np.uint64).reshape(B)
    D = R - B
    res = SampleResult(np.full(B, -2, np.int32), np.full(R, -1, np.int32), np.full((D, 2), np.nan),
                       np.full(D, np.nan), np.full(R, np.nan), np.full(R, np.nan), np.full(D, np.inf),
                       np.full(B, np.inf), np.full(B, np.nan), np.full(D, np.nan))
    for b in _rows_arg(rows, B):
        t0, kb, ok = seqs[b]
        if not ok:
            res.accepted_len[b] = -1
            continue
        s = accept_sample(z[None, t0:t0 + kb + 1], zd[None, t0 - b:t0 - b + kb], d[None, t0 - b:t0 - b + kb],
                          temperature, seeds[b:b + 1], slots=[b])
        tr, dr = slice(t0, t0 + kb + 1), slice(t0 - b, t0 - b + kb)
        res.accepted_len[b] = s.accepted_len[0]
        res.out_tokens[tr] = s.out_tokens[0]
        res.u_accept[tr], res.u_terminal[tr] = s.u_accept[0], s.u_terminal[0]
        res.probs_at_draft[dr] = s.probs_at_draft[0]
        res.ratio[dr], res.accept_margin[dr], res.alpha[dr] = s.ratio[0], s.accept_margin[0], s.alpha[0]
        res.terminal_margin[b], res.residual_mass[b] = s.terminal_margin[0], s.residual_mass[0]
    return res


# ------------------------------------------------ expected tokens per pass --

def expected_tokens(alpha: float, K: int) -> float:
    """(1 - alpha^(K+1)) / (1 - alpha): expected tokens per verify pass when
    every draft is accepted independently with probability alpha
    ("Inference-4", The idea; "speculative-decoding" blog, Why speculative
    decoding is fast).  Limits: alpha = 1 gives K + 1, alpha = 0 gives 1."""
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def expected_tokens_positional(alphas) -> float:
    """sum_{i=0}^{K} prod_{j<i} alpha_j: the same expectation when the accept
    probability differs per position (each term is the probability of
    reaching position i)."""
    total, reach = 1.0, 1.0
    for a in alphas:
        reach *= a
        total += reach
    return total
