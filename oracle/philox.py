"""Philox4x32-10 counter-based generator — oracle side (test infrastructure).

None of the three pages names a generator; both sides of the verify step must
draw identical uniforms, so each implements one counter-based generator from
its published definition: Philox4x32 with 10 rounds, J. K. Salmon, M. A.
Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
SC'11, section 3 (the Philox S-box: two 32x32->64 multiplies per round, the
high halves xored with the other counter words and the round key, the round
key advanced by a Weyl sequence between rounds).

Written with numpy uint64 arithmetic so that it applies elementwise to arrays
of counters; scalar Python ints work too.
"""

import numpy as np

PHILOX_ROUNDS = 10

# Round multipliers and Weyl key increments of Philox4x32 (SC'11, section 3).
_MUL0 = np.uint64(0xD2511F53)
_MUL1 = np.uint64(0xCD9E8D57)
_WEYL0 = np.uint64(0x9E3779B9)
_WEYL1 = np.uint64(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words for counter (c0..c3) and key (k0, k1).

    Each round: the products of the multipliers with counter words 0 and 2
    are split into high and low halves; the new counter is
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
    then advances by the Weyl constants.  Ten rounds.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    for _ in range(PHILOX_ROUNDS):
        prod0 = _MUL0 * c0
        prod1 = _MUL1 * c2
        hi0, lo0 = prod0 >> _SHIFT32, prod0 & _MASK32
        hi1, lo1 = prod1 >> _SHIFT32, prod1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
        k0 = (k0 + _WEYL0) & _MASK32
        k1 = (k1 + _WEYL1) & _MASK32
    return c0, c1, c2, c3


def uniforms(seed, request, position, step):
    """Two uniforms in [0, 1) for one (request, draft position, step).

    Key = (low, high) 32-bit halves of the 64-bit seed; counter =
    (request, position, step low, step high).  u comes from output word 0 and
    v from word 1, each keeping its top 24 bits: (word >> 8) * 2**-24, which
    is exact in fp32 and fp64.  u drives the accept test at that position and
    v drives the token draw made at that position (residual or bonus).
    Arrays broadcast.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    step = int(step) & 0xFFFFFFFFFFFFFFFF
    x0, x1, _, _ = philox4x32_10(request, position, step & 0xFFFFFFFF, step >> 32,
                                 seed & 0xFFFFFFFF, seed >> 32)
    scale = 2.0 ** -24
    u = (x0 >> np.uint64(8)).astype(np.float64) * scale
    v = (x1 >> np.uint64(8)).astype(np.float64) * scale
    if u.ndim == 0:
        return float(u), float(v)
    return u, v
