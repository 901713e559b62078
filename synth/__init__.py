"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only *draws* inputs: LM-head weights, hidden states, draft
logits, draft tokens, per-sequence seeds and per-row greedy/sampled flags.
It holds none of the verify step's own arithmetic (no softmax statistics, no
acceptance rule, no residual sampling), so that the GPU path and the CPU
oracle, which both consume these inputs, share no code beyond them.

Two inputs are built from a quick fp32 product of the drawn hidden states and
weights ("base logits"): the draft logits are defined by the workloads as the
target logits plus noise (or reweighted by rank).  The base logits are only a
device to correlate draft with target; neither side's result is checked
against them, and both sides receive the same frozen draft logits.

Drafts for sampled rows are drawn from the draft distribution softmax(z_d/T)
by the Gumbel-max construction (argmax of z_d/T plus Gumbel noise); drafts for
greedy rows are argmax z_d.  Speculative sampling requires the drafts to come
from the draft distribution ("Inference-4", Draft-model speculative decoding,
sampling bullet); greedy drafting takes the draft's most likely token (same
page, the DraftModel listing).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "weights", "hidden_states", "base_logits",
    "draft_logits", "sampled_mask", "draft_tokens", "seeds", "round_inputs",
    "draft_counts", "row_start", "pack_rows", "tree_parents", "tree_tokens",
    "NgramWorkload", "NGRAM_WORKLOADS", "histories",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic verify workload.

    B sequences, K drafts each (K+1 verify positions), hidden size H,
    vocabulary V.  ``dtype`` is the storage type of hidden states and LM-head
    weights ("f32" or "bf16"; bf16 values are drawn in fp32 and rounded to
    nearest-even before either side sees them).
    """
    name: str
    B: int
    K: int
    H: int
    V: int
    dtype: str
    w_std: float
    temperature: float
    draft: str                 # "additive" | "scaled" | "zipf"
    draft_sigma: tuple = (1.0, 1.0)   # (lo, hi): per-row sigma ~ U[lo, hi]
    draft_scale: float = 1.0          # "scaled": z_d = scale * z + N(0, sigma)
    zipf_s: float = 1.1               # "zipf": p_d ∝ q_t * rank^-s
    modes: str = "sample"      # "sample" | "greedy" | "both" | "half" | "bernoulli"
    data_seed: int = 1000
    ragged: bool = False       # per-sequence draft counts K_b ~ U{0..K}, rows packed
    tree: bool = False         # K = N draft nodes per sequence in a random tree
    note: str = field(default="", compare=False)

    @property
    def M(self) -> int:
        return self.B * (self.K + 1)


# The five workloads of the benchmark description, with the readings of
# unstated details (weight std of the 64- and 512-sequence cases, which half
# is greedy, the Zipf reweighting by target rank) written out in the design
# notes.
WORKLOADS = {
    "tiny_b1_k4_h256_v1000": Workload(
        "tiny_b1_k4_h256_v1000", B=1, K=4, H=256, V=1000, dtype="f32",
        w_std=0.05, temperature=1.0, draft="additive", draft_sigma=(1.0, 1.0),
        modes="both", data_seed=1000,
        note="fp32, both modes, Philox seed = round, hidden and noise redrawn per round"),
    "b1_k5_h4096_v128256": Workload(
        "b1_k5_h4096_v128256", B=1, K=5, H=4096, V=128256, dtype="bf16",
        w_std=0.02, temperature=1.0, draft="additive", draft_sigma=(0.5, 0.5),
        modes="sample", data_seed=1001,
        note="sampled at T=1, seeds 0..9999"),
    "b64_k4_h4096_v128256": Workload(
        "b64_k4_h4096_v128256", B=64, K=4, H=4096, V=128256, dtype="bf16",
        w_std=0.02, temperature=0.8, draft="additive", draft_sigma=(0.0, 2.0),
        modes="half", data_seed=1002,
        note="rows 0..31 greedy, 32..63 sampled at T=0.8"),
    "b256_k8_h8192_v152064": Workload(
        "b256_k8_h8192_v152064", B=256, K=8, H=8192, V=152064, dtype="bf16",
        w_std=0.015, temperature=0.7, draft="scaled", draft_sigma=(1.0, 1.0),
        draft_scale=0.7, modes="sample", data_seed=1003),
    "b512_k3_h5120_v262144": Workload(
        "b512_k3_h5120_v262144", B=512, K=3, H=5120, V=262144, dtype="bf16",
        w_std=0.02, temperature=1.0, draft="zipf", modes="bernoulli",
        data_seed=1004),
    # long verify blocks (not one of the five benchmark workloads): 16-token
    # blocks (K = 15) at 32 concurrent sequences, the LM-head shape of the
    # 8B-parameter target the pages measure block drafting on
    "b32_k15_h4096_v151936": Workload(
        "b32_k15_h4096_v151936", B=32, K=15, H=4096, V=151936, dtype="bf16",
        w_std=0.02, temperature=1.0, draft="additive", draft_sigma=(0.5, 0.5),
        modes="half", data_seed=1008,
        note="K = 15 blocks at B = 32; rows 0..15 greedy, 16..31 sampled at T=1"),
    # per-sequence draft counts (not one of the five benchmark workloads): the
    # 64-sequence mixed batch with K_b drawn uniformly from 0..7
    "b64_k0to7_h4096_v128256": Workload(
        "b64_k0to7_h4096_v128256", B=64, K=7, H=4096, V=128256, dtype="bf16",
        w_std=0.02, temperature=0.8, draft="additive", draft_sigma=(0.0, 2.0),
        modes="half", data_seed=1005, ragged=True,
        note="K_b ~ U{0..7}, packed rows; rows 0..31 greedy, 32..63 sampled at T=0.8"),
    # draft trees (not one of the five benchmark workloads): 8 sequences with
    # 63-node trees, greedy
    "b8_tree63_h4096_v128256": Workload(
        "b8_tree63_h4096_v128256", B=8, K=63, H=4096, V=128256, dtype="bf16",
        w_std=0.02, temperature=1.0, draft="additive", draft_sigma=(0.05, 0.05),
        modes="greedy", data_seed=1006, tree=True,
        note="63-node random trees; children take the parent's top-k tokens under N(0, 0.05^2) noise"),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _tdtype(wl: Workload):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def weights(wl: Workload, device="cpu", seed: int | None = None) -> torch.Tensor:
    """LM-head weights W[V, H], N(0, w_std^2), stored in ``wl.dtype``.

    Drawn in row blocks so that a bf16 draw never holds the whole fp32 matrix.
    """
    seed = wl.data_seed if seed is None else seed
    g = _gen(seed * 7919 + 1, device)
    out = torch.empty((wl.V, wl.H), dtype=_tdtype(wl), device=device)
    rows = max(1, (1 << 26) // max(wl.H, 1))
    for v0 in range(0, wl.V, rows):
        v1 = min(wl.V, v0 + rows)
        blk = torch.randn((v1 - v0, wl.H), generator=g, device=device, dtype=torch.float32)
        out[v0:v1] = (blk * wl.w_std).to(out.dtype)
    return out


def hidden_states(wl: Workload, device="cpu", rnd: int = 0) -> torch.Tensor:
    """Hidden states at the K+1 verify positions, [B, K+1, H], N(0, 1)."""
    g = _gen(wl.data_seed * 1_000_003 + 17 * rnd + 2, device)
    x = torch.randn((wl.B, wl.K + 1, wl.H), generator=g, device=device, dtype=torch.float32)
    return x.to(_tdtype(wl))


def base_logits(hidden: torch.Tensor, W: torch.Tensor, chunk: int = 32768) -> torch.Tensor:
    """fp32 product hidden·Wᵀ, [B, K+1, V], used only to correlate the draft
    logits with the target (see the module docstring)."""
    B, P, H = hidden.shape
    x = hidden.reshape(B * P, H).float()
    V = W.shape[0]
    out = torch.empty((B * P, V), dtype=torch.float32, device=hidden.device)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        out[:, v0:v1] = x @ W[v0:v1].float().t().contiguous()
    return out.reshape(B, P, V)


def draft_logits(wl: Workload, base: torch.Tensor, rnd: int = 0) -> torch.Tensor:
    """Draft logits z_d[B, K, V] (fp32) built from the base logits at the K
    draft positions, following the workload's recipe."""
    B, K, V = wl.B, wl.K, wl.V
    dev = base.device
    if K == 0:
        return torch.empty((B, 0, V), dtype=torch.float32, device=dev)
    z = base[:, :K, :].float()
    g = _gen(wl.data_seed * 1_000_033 + 31 * rnd + 3, dev)
    if wl.draft == "additive":
        lo, hi = wl.draft_sigma
        if lo == hi:
            sig = torch.full((B, 1, 1), float(lo), device=dev)
        else:
            sig = (lo + (hi - lo) * torch.rand((B, 1, 1), generator=g, device=dev))
        return z + sig * torch.randn(z.shape, generator=g, device=dev)
    if wl.draft == "scaled":
        return wl.draft_scale * z + wl.draft_sigma[0] * torch.randn(z.shape, generator=g, device=dev)
    if wl.draft == "zipf":
        # rank 1 = largest base logit, ties broken by lower index (stable sort)
        order = torch.sort(z, dim=-1, descending=True, stable=True).indices
        rank = torch.empty_like(order)
        ar = torch.arange(1, V + 1, device=dev).expand_as(order)
        rank.scatter_(-1, order, ar)
        return z - wl.zipf_s * torch.log(rank.float()) * wl.temperature
    raise ValueError(wl.draft)


def sampled_mask(wl: Workload, rnd: int = 0) -> np.ndarray:
    """Boolean [B]: True where the row verifies in sampled mode."""
    B = wl.B
    if wl.modes == "sample":
        return np.ones(B, bool)
    if wl.modes == "greedy":
        return np.zeros(B, bool)
    if wl.modes == "half":
        return np.arange(B) >= B // 2
    if wl.modes == "both":
        # the same row is verified once in each mode; callers pick the mode
        return np.ones(B, bool)
    if wl.modes == "bernoulli":
        rs = np.random.default_rng(wl.data_seed * 7 + rnd)
        return rs.random(B) < 0.5
    raise ValueError(wl.modes)


def draft_tokens(zd: torch.Tensor, sampled: np.ndarray, temperature: float, seed: int) -> torch.Tensor:
    """Draft tokens [B, K] int32: Gumbel-max draws from softmax(z_d/T) for
    sampled rows, argmax z_d for greedy rows."""
    B, K, V = zd.shape
    dev = zd.device
    if K == 0:
        return torch.empty((B, 0), dtype=torch.int32, device=dev)
    g = _gen(seed, dev)
    u = torch.rand(zd.shape, generator=g, device=dev, dtype=torch.float64)
    u = u.clamp_(min=1e-300)
    gumbel = -torch.log(-torch.log(u))
    samp = torch.argmax(zd.double() / temperature + gumbel, dim=-1)
    greedy = torch.argmax(zd, dim=-1)
    m = torch.as_tensor(sampled, device=dev).view(B, 1)
    return torch.where(m, samp, greedy).to(torch.int32)


def seeds(wl: Workload, rnd: int = 0) -> np.ndarray:
    """Per-sequence Philox seeds for one verify round: seed_b = rnd*B + b."""
    return (np.uint64(rnd) * np.uint64(wl.B) + np.arange(wl.B, dtype=np.uint64)).astype(np.uint64)


def round_inputs(wl: Workload, rnd: int = 0, device="cpu", W: torch.Tensor | None = None,
                 hidden: torch.Tensor | None = None):
    """All inputs of one verify round (W and hidden may be passed in to keep
    them fixed across rounds)."""
    if W is None:
        W = weights(wl, device)
    if hidden is None:
        hidden = hidden_states(wl, device, rnd)
    base = base_logits(hidden, W)
    zd = draft_logits(wl, base, rnd)
    smask = sampled_mask(wl, rnd)
    d = draft_tokens(zd, smask, wl.temperature, seed=wl.data_seed * 104729 + rnd)
    return dict(W=W, hidden=hidden, draft_logits=zd, sampled=smask, drafts=d,
                seeds=seeds(wl, rnd), temperature=wl.temperature)



# ------------------------------------------------ per-sequence draft counts --

def draft_counts(B: int, K_max: int, seed: int) -> np.ndarray:
    """Per-sequence draft counts K_b ~ U{0..K_max}, int32 [B]."""
    return np.random.default_rng(seed).integers(0, K_max + 1, B).astype(np.int32)


def row_start(counts) -> np.ndarray:
    """Packing offsets [B+1] int32: row_start[0] = 0, row_start[b+1] =
    row_start[b] + K_b + 1 (target rows of sequence b)."""
    c = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(c + 1)]).astype(np.int32)


def pack_rows(dense, counts, drafts: bool = False):
    """Concatenate, in sequence order, the first K_b + 1 (target rows) or K_b
    (``drafts``) entries along axis 1 of a dense [B, P, ...] array or tensor."""
    keep = [int(k) + (0 if drafts else 1) for k in np.asarray(counts)]
    parts = [dense[b, :keep[b]] for b in range(len(keep))]
    if isinstance(dense, torch.Tensor):
        return torch.cat(parts, dim=0) if parts else dense.reshape(0, *dense.shape[2:])
    return np.concatenate(parts, axis=0)


# ----------------------------------------------------------- draft trees --

def tree_parents(B: int, N: int, seed: int) -> np.ndarray:
    """Random tree shapes [B, N+1] int32 in topological order: node v >= 1
    hangs under v - g, g >= 1 geometric(0.45) (clipped at the root), so trees
    mix long chains with branches; entry 0 (the root) is 0."""
    rng = np.random.default_rng(seed)
    par = np.zeros((B, N + 1), np.int64)
    for v in range(1, N + 1):
        g = rng.geometric(0.45, B)
        par[:, v] = np.maximum(v - g, 0)
    return par.astype(np.int32)


def tree_tokens(node_logits: torch.Tensor, parents, seed: int, p_random: float = 0.25,
                sigma: float = 1.0) -> torch.Tensor:
    """Draft tokens of tree nodes [B, N+1] int32 (entry 0 unused): the j-th
    child of a node takes the j-th most likely token of a copy of the parent's
    logits with N(0, sigma^2) noise added (a top-k expansion), or a uniform
    random token with probability p_random."""
    B, P, V = node_logits.shape
    par = np.asarray(parents, np.int64)
    rank = np.zeros((B, P), np.int64)
    for b in range(B):
        seen = {}
        for v in range(1, P):
            p = par[b, v]
            rank[b, v] = seen.get(p, 0)
            seen[p] = rank[b, v] + 1
    kmax = int(rank.max()) + 1 if P > 1 else 1
    g = _gen(seed, node_logits.device)
    noisy = node_logits.float() + sigma * torch.randn(node_logits.shape, generator=g, device=node_logits.device)
    top = torch.topk(noisy, min(kmax, V), dim=-1).indices.cpu().numpy()     # [B, P, kmax]
    rs = np.random.default_rng(seed)
    tok = np.zeros((B, P), np.int64)
    for v in range(1, P):
        tok[:, v] = top[np.arange(B), par[:, v], np.minimum(rank[:, v], top.shape[-1] - 1)]
    rnd = rs.random((B, P)) < p_random
    tok = np.where(rnd, rs.integers(0, V, (B, P)), tok)
    tok[:, 0] = 0
    return torch.from_numpy(tok.astype(np.int32))


# ------------------------------------------------ prompt-lookup histories --

@dataclass(frozen=True)
class NgramWorkload:
    """Token histories for the prompt-lookup drafter: B sequences of length
    U[L/2, L] over a vocabulary of V tokens, built from fresh random tokens
    and copies of earlier spans (copy-heavy text such as summarisation or
    retrieval answers, where the pages say prompt lookup pays)."""
    name: str
    B: int
    L: int
    V: int
    max_ngram: int
    n_drafts: int
    copy_frac: float
    data_seed: int


NGRAM_WORKLOADS = {
    "ngram_b256_l131072": NgramWorkload("ngram_b256_l131072", B=256, L=131072, V=128256, max_ngram=3, n_drafts=7,
                                        copy_frac=0.5, data_seed=1007),
}


def histories(B: int, L: int, V: int, seed: int, copy_frac: float = 0.5, lengths=None) -> list:
    """B int32 token histories.  Lengths U[L/2, L] unless given.  Start from
    uniform random tokens, then copy spans of 8..64 tokens from earlier
    positions over about copy_frac of the sequence; with probability
    copy_frac the sequence ends inside a copied span."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(L // 2, L + 1, B)
    out = []
    for b in range(B):
        n = int(lengths[b])
        s = rng.integers(0, V, n).astype(np.int32)
        if n > 16:
            n_copies = int(copy_frac * n / 36)
            dst = np.sort(rng.integers(8, n, n_copies))
            ln = rng.integers(8, 65, n_copies)
            for d, k in zip(dst, ln):
                src = int(rng.integers(0, d - 4))
                k = int(min(k, n - d, d - src))
                s[d:d + k] = s[src:src + k]
            if rng.random() < copy_frac:
                k = int(min(rng.integers(8, 65), n // 2))
                src = int(rng.integers(0, n - k - k // 2 + 1)) if n - k - k // 2 > 0 else 0
                s[n - k:] = s[src:src + k]
        out.append(s)
    return out
