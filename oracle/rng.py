"""Counter-based random numbers for stochastic rounding (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Stochastic rounding needs random bits that both the device and the oracle can
produce for any element independently, so the generator is a counter-based
one: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC 2011), written here from its published definition and
pinned by the published known-answer vectors (tests/golden/philox4x32_10_kat.txt).

One round maps the counter (c0, c1, c2, c3) with key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)),
M0 = 0xD2511F53, M1 = 0xCD9E8D57 (32x32 -> 64-bit products); the key is bumped by
the Weyl constants (0x9E3779B9, 0xBB67AE85) between rounds; 10 rounds.
"""

from __future__ import annotations

import numpy as np

M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
W0, W1 = np.uint32(0x9E3779B9), np.uint32(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr: uint32 array (..., 4); key: uint32 array (..., 2) (broadcast). Returns uint32 (..., 4)."""
    c = [np.asarray(ctr, dtype=np.uint32)[..., i].astype(np.uint64) for i in range(4)]
    k0 = np.asarray(key, dtype=np.uint32)[..., 0].astype(np.uint64)
    k1 = np.asarray(key, dtype=np.uint32)[..., 1].astype(np.uint64)
    for rnd in range(10):
        p0 = M0 * c[0]                                   # < 2^64: exact in uint64
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        if rnd < 9:
            k0 = (k0 + np.uint64(W0)) & MASK32
            k1 = (k1 + np.uint64(W1)) & MASK32
    return np.stack([x.astype(np.uint32) for x in c], axis=-1)


def element_words(seed: int, idx) -> np.ndarray:
    """The 32-bit random word of element `idx` (an index into a tensor, row-major):
    word idx % 4 of Philox4x32-10 with counter (idx // 4 low 32 bits, high 32 bits, 0, 0)
    and key (seed low 32 bits, high 32 bits)."""
    idx = np.asarray(idx, dtype=np.uint64)
    blk = idx >> np.uint64(2)
    ctr = np.stack([(blk & MASK32).astype(np.uint32), (blk >> np.uint64(32)).astype(np.uint32),
                    np.zeros(blk.shape, np.uint32), np.zeros(blk.shape, np.uint32)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    out = philox4x32_10(ctr, key)
    return np.take_along_axis(out, (idx & np.uint64(3)).astype(np.int64)[..., None], axis=-1)[..., 0]
