"""Philox4x32-10, written from its published definition.

Source: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11: the Philox construction and its table of round
multipliers and Weyl key increments for the 4x32 variant.

One round maps a 4-word counter (c0, c1, c2, c3) under a 2-word key (k0, k1):

    hi0:lo0 = M0 * c0        (full 64-bit product of two 32-bit words)
    hi1:lo1 = M1 * c2
    out     = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)

and between rounds the key is bumped by the Weyl constants (k0 += W0,
k1 += W1, mod 2^32).  Philox4x32-10 applies ten rounds, the first with the
key as given.  Everything here is vectorised over numpy arrays of uint32.

Part of the oracle (test infrastructure); see oracle/__init__.py.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(counter, key):
    """Raw Philox4x32-10 blocks.

    counter: uint32 array of shape (..., 4); key: uint32 array (..., 2)
    (broadcastable).  Returns uint32 (..., 4).
    """
    c = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> _SH, p0 & _MASK
        hi1, lo1 = p1 >> _SH, p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    out = np.stack(np.broadcast_arrays(c0, c1, c2, c3), axis=-1)
    return out.astype(np.uint32)


def uniform24(word):
    """Map a 32-bit word to [0, 1) on the 24-bit grid: (word >> 8) * 2^-24.

    Every value is exact in both fp32 and fp64.
    """
    w = np.asarray(word, dtype=np.uint32)
    return (w >> np.uint32(8)).astype(np.float64) * (2.0 ** -24)


def verify_uniforms(seed, seq, pos):
    """The two uniforms the verify step draws for sequence slot ``seq`` at
    verify position ``pos`` under per-sequence ``seed`` (uint64).

    Counter = (pos, seq, 0, 0); key = (low 32 bits of seed, high 32 bits).
    Word 0 drives the accept test, word 1 the terminal (residual or bonus)
    draw.  Returns (u_accept, u_terminal) as float64 arrays.
    """
    seed = np.asarray(seed, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    seq = np.asarray(seq, dtype=np.uint64)
    seed, seq, pos = np.broadcast_arrays(seed, seq, pos)
    ctr = np.stack([pos & _MASK, seq & _MASK, np.zeros_like(pos), np.zeros_like(pos)], axis=-1)
    key = np.stack([seed & _MASK, seed >> _SH], axis=-1)
    blk = philox4x32_10(ctr, key)
    return uniform24(blk[..., 0]), uniform24(blk[..., 1])
