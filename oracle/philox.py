"""Philox4x64-10 in plain Python integers (test infrastructure only).

Definition: Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
as 1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds.  One round
multiplies counter words 0 and 2 by two fixed odd constants, keeps the high
and low halves of the 128-bit products, and mixes the high halves with
counter words 1 and 3 and the two key words; between rounds the key is
bumped by two Weyl constants.  The constants are the published ones for
the 4x64 variant.

Pin: tests/test_philox.py checks raw words against numpy.random.Philox,
which implements the same generator (4x64, 10 rounds).
"""

from __future__ import annotations

_MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(ctr, key):
    """Return the 4 output words (Python ints) for counter ``ctr`` (4 words) and ``key`` (2 words)."""
    c0, c1, c2, c3 = (int(c) & _MASK64 for c in ctr)
    k0, k1 = (int(k) & _MASK64 for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & _MASK64
            k1 = (k1 + PHILOX_W1) & _MASK64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 64, p0 & _MASK64
        hi1, lo1 = p1 >> 64, p1 & _MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform24(word):
    """Top 24 bits of a 64-bit word as an exact dyadic in [0, 1)."""
    return float((int(word) >> 40)) * 2.0 ** -24


def uniform53(word):
    """Top 53 bits of a 64-bit word as an exact dyadic in [0, 1)."""
    return float((int(word) >> 11)) * 2.0 ** -53
