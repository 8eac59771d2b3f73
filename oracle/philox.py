"""Philox4x32-10 counter-based generator.  TEST INFRASTRUCTURE ONLY.

Written from its published definition (J. Salmon, M. Moraes, R. Dror,
D. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11, section on
the Philox S-box): a 4-word counter and a 2-word key; each of the 10 rounds
multiplies counter words 0 and 2 by two fixed 32-bit multipliers, splits each
64-bit product into high and low halves, and forms the new counter from the
halves XORed with the other two words and the key; the key is advanced by two
fixed Weyl increments between rounds.

The pages name no generator; the sampler only needs one uniform per
(batch, head, query block, KV block), and a counter-based one gives the same
value on the CPU and the GPU without shared state.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32 with 10 rounds.

    Counter words c0..c3 and key words k0, k1 are arrays (or scalars)
    broadcastable to a common shape, values in [0, 2^32). Returns four uint64
    arrays holding 32-bit output words.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c0                      # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3
