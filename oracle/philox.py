"""Philox4x64-10 counter-based generator (oracle side).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
(SC'11), the Philox-4x64 bijection with 10 rounds.  State: four 64-bit counter words
c0..c3 and two 64-bit key words k0, k1.  One round multiplies c0 and c2 by two fixed
odd constants, keeps the 128-bit products as (hi, lo) pairs, and permutes:
    (c0, c1, c2, c3) <- (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
after which the key is bumped by two Weyl constants (the golden ratio and sqrt(3) - 1
as 64-bit fractions).  Ten rounds with nine key bumps in between.

The pages name no generator.  Reading taken: the draws of the acceptance test and of
the correction/bonus sampler are keyed by (seed, sequence, position, step offset) so
that any independent implementation reproduces them; Philox4x64-10 is used because
numpy ships an independent implementation of it to pin against.

Pinned by tests/test_oracle_philox.py against ``numpy.random.Philox``.
"""
from __future__ import annotations

_MASK64 = (1 << 64) - 1
_M0 = 0xD2E7470EE14C6C93
_M1 = 0xCA5A826395121157
_W0 = 0x9E3779B97F4A7C15
_W1 = 0xBB67AE8584CAA73B

# 24-bit uniforms: every value k * 2^-24 is exact in float32 and float64.
_U24 = 1.0 / (1 << 24)


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for a 4-word counter and a 2-word key."""
    c0, c1, c2, c3 = (int(x) & _MASK64 for x in counter)
    k0, k1 = (int(x) & _MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK64
            k1 = (k1 + _W1) & _MASK64
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & _MASK64,
                          (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64)
    return c0, c1, c2, c3


def uniforms(seed: int, seq: int, pos: int, offset: int = 0):
    """(u_acc, u_smp) for one draft position.

    Counter = (pos, seq, offset, 0), key = (seed, 0).  u_acc is the top 24 bits of word
    0, u_smp the top 24 bits of word 1, each scaled by 2^-24 into [0, 1 - 2^-24].
    ``pos`` is the draft position j (linear) or the node index (tree).
    """
    w0, w1, _, _ = philox4x64_10((pos, seq, offset, 0), (seed, 0))
    return (w0 >> 40) * _U24, (w1 >> 40) * _U24
