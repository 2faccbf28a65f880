"""Philox4x64-10 counter-based generator and the uniforms drawn from it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the published definition (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11): a 4-word 64-bit counter and a
2-word key; ten rounds, each multiplying words 0 and 2 by the round constants
into 128-bit products, permuting, and xoring the high halves with the other
two words and the key; the key is bumped by the Weyl constants between
rounds.

Stream layout used by the stochastic accept (key = (seed, 0)):
counter = (round, slot, stream, 0) with stream 0 = draft sample, 1 = accept
test, 2 = residual / bonus sample.  A uniform is the top 24 bits of output
word 0 times 2^-24, exactly representable in float32.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B

STREAM_DRAFT = 0
STREAM_ACCEPT = 1
STREAM_RESAMPLE = 2


def philox4x64_10(counter, key):
    """Return the 4 output words for a 4-word counter and 2-word key."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for _ in range(10):
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & MASK64
        k1 = (k1 + PHILOX_W1) & MASK64
    return x0, x1, x2, x3


def uniform24(word: int) -> float:
    """Map a 64-bit word to [0, 1) with 24 bits (exact in float32)."""
    return float((int(word) >> 40) & 0xFFFFFF) * (2.0 ** -24)


def uniform(seed: int, rnd: int, slot: int, stream: int) -> float:
    return uniform24(philox4x64_10((rnd, slot, stream, 0), (seed, 0))[0])
