"""Philox4x32-10 counter-based generator, for the dropout oracle (test infrastructure only).

The generator of Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
easy as 1, 2, 3" (SC'11), as defined there: a 128-bit counter (four 32-bit
words) and a 64-bit key (two words) go through ten rounds.  In a round, the
words c0 and c2 are multiplied by the two Philox multipliers into 64-bit
products; the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3
^ k1, lo(M0 c0)); between rounds the key is bumped by the two Weyl
constants.  The multipliers and Weyl constants are the published ones.

The dropout rule built on it (the "StreamAttention" page names deterministic
Philox seeding for dropout in "Recent Updates"; the counter layout and the
16-bit decisions are a reading of this repository): each generator block
gives eight 16-bit values, one per decision.  The probability of query row
i, key j in (batch b, head h) is decided by 16-bit half ``(j % 64) // 32``
(0 = low, 1 = high) of word ``j % 4`` of the block with counter
``(8 (j // 64) + (j % 32) // 4, i, b * H_q + h, offset)`` and key
``(seed_lo, seed_hi)``: within each window of 64 keys, keys j and j + 32
share a word.  It is kept when that value is at least ``drop_threshold(p)``
= floor(p 2^16), so the drop probability is p rounded down to a multiple of
2^-16.

``philox4x32_10`` works on Python ints one block at a time; ``philox_words``
is the same arithmetic vectorised over numpy uint64 arrays.
"""
from __future__ import annotations

import math

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57   # round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85   # key schedule (Weyl) increments
MASK32 = 0xFFFFFFFF
ROUNDS = 10


def philox4x32_10(ctr, key):
    """One block: ``ctr`` four 32-bit ints, ``key`` two; returns four ints."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in ctr)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(ROUNDS):
        if r:
            k0, k1 = (k0 + W0) & MASK32, (k1 + W1) & MASK32
        p0, p1 = M0 * c0, M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK32, p1 & MASK32, ((p0 >> 32) ^ c3 ^ k1) & MASK32, p0 & MASK32
    return c0, c1, c2, c3


def philox_words(c0, c1, c2, c3, k0, k1):
    """Vectorised blocks: counter words as broadcastable integer arrays, key as
    two ints.  Returns the four output words as uint64 arrays (values < 2^32)."""
    m = np.uint64(MASK32)
    c = [np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (x.copy() for x in c)
    k0, k1 = int(k0) & MASK32, int(k1) & MASK32
    for r in range(ROUNDS):
        if r:
            k0, k1 = (k0 + W0) & MASK32, (k1 + W1) & MASK32
        p0 = c0 * np.uint64(M0)
        p1 = c2 * np.uint64(M1)
        c0, c1, c2, c3 = (((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)) & m, p1 & m,
                          ((p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)) & m, p0 & m)
    return c0, c1, c2, c3


def drop_threshold(p):
    """16-bit values below this threshold drop: floor(p * 2^16), for 0 <= p < 1."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(math.floor(float(p) * 2.0 ** 16)), 0xFFFF)


def decision_slot(j):
    """(block counter word c0, word, half) of key j's decision."""
    return 8 * (j // 64) + (j % 32) // 4, j % 4, (j % 64) // 32


def dropout_values(b, h, H_q, rows, S_k, seed, offset=0):
    """The 16-bit decision values ``[R, S_k]`` (uint64) of (batch b, head h)
    for query rows ``rows``."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(S_k, dtype=np.int64)
    c0, word, half = decision_slot(j)
    words = philox_words(c0[None, :], rows[:, None], b * H_q + h, offset,
                         seed & MASK32, (seed >> 32) & MASK32)
    w = np.choose(word[None, :].repeat(len(rows), axis=0), words)
    return (w >> (np.uint64(16) * half.astype(np.uint64))[None, :]) & np.uint64(0xFFFF)


def keep_mask(b, h, H_q, rows, S_k, p, seed, offset=0):
    """Boolean ``[R, S_k]`` keep decisions of (batch b, head h) for query rows ``rows``."""
    return dropout_values(b, h, H_q, rows, S_k, seed, offset) >= np.uint64(drop_threshold(p))
