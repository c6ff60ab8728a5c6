"""Philox4x32-10 counter-based generator, for the dropout keep bits -- TEST INFRASTRUCTURE ONLY.

Written from the published definition (Salmon, Moraes, Dror, Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC 2011, the Philox family): a 4 x 32-bit counter and a
2 x 32-bit key; each round multiplies counter words 0 and 2 by the two Philox
multipliers (64-bit products split into high and low halves), mixes the high halves
with the other two counter words and the key by XOR, and permutes the words; between
rounds the key is advanced by the two Weyl constants. Ten rounds. numpy uint64
arithmetic keeps every product exact. Vectorised over any number of counters.

Pinned by the authors' published known-answer vectors (tests/golden/philox4x32_10_kat.json).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(ctr, key, rounds: int = 10):
    """ctr: uint32-valued array [..., 4]; key: [..., 2] (broadcast). Returns uint32 [..., 4]."""
    c = np.asarray(ctr, dtype=np.uint64) & MASK32
    k = np.broadcast_to(np.asarray(key, dtype=np.uint64) & MASK32, c.shape[:-1] + (2,))
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c0  # < 2^64: exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)
