"""Philox4x32-10 and the maps from its output words to uniforms and Gumbels.

Test infrastructure only (see the package docstring).

The pages say nothing about how random numbers are drawn.  Both sides of the
comparison therefore implement one published counter-based generator, Philox4x32
with 10 rounds, from its definition in J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (section on the
Philox family): a 4-word counter and a 2-word key; each round multiplies words 0
and 2 by two fixed odd constants, keeps both halves of the 64-bit products, and
mixes the high halves with words 1 and 3 and the round key; the key is advanced
by two Weyl constants between rounds.

Counter layout of one draw (the reading of the pages taken here):
    key     = (seed mod 2^32, seed div 2^32)
    counter = (n div 4, position, request, stream)
    word    = n mod 4 of the four output words
where n is the index of the draw inside its stream (a block, tile or element
index of the sampler), position = block position + the request's position
offset, and stream names which decision of the round the draw feeds.
"""

from __future__ import annotations

import numpy as np

# Multipliers and Weyl increments of Philox4x32 (SC'11).
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)

# Streams: which decision a draw belongs to.
DRAFT_TOP, DRAFT_MID, DRAFT_LEAF = 0, 1, 2
ACCEPT = 3
FINAL_TOP, FINAL_MID, FINAL_LEAF = 4, 5, 6


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Ten Philox4x32 rounds on counter words (c0..c3) (broadcastable uint32
    arrays) under key (k0, k1).  Returns the four output words as uint32 arrays."""
    x = [np.asarray(c, dtype=np.uint64) & _LO for c in (c0, c1, c2, c3)]
    x = list(np.broadcast_arrays(*x))
    ka, kb = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            ka = (ka + _W0) & 0xFFFFFFFF
            kb = (kb + _W1) & 0xFFFFFFFF
        p0 = _M0 * x[0]
        p1 = _M1 * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _LO
        hi1, lo1 = p1 >> np.uint64(32), p1 & _LO
        x = [hi1 ^ x[1] ^ np.uint64(ka), lo1, hi0 ^ x[3] ^ np.uint64(kb), lo0]
    return [w.astype(np.uint32) for w in x]


def words(seed: int, stream: int, request: int, position: int, count: int) -> np.ndarray:
    """The first ``count`` 32-bit draws of one (stream, request, position)."""
    n = np.arange(count, dtype=np.uint64)
    out = philox4x32_10(n // np.uint64(4), np.uint64(position & 0xFFFFFFFF),
                        np.uint64(request & 0xFFFFFFFF), np.uint64(stream),
                        seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    lane = (n % np.uint64(4)).astype(np.int64)
    return np.choose(lane, out)


def to_uniform(w: np.ndarray) -> np.ndarray:
    """u = (floor(w / 2^9) + 1/2) * 2^-23: the 2^23 odd multiples of 2^-24 in
    (0, 1).  Every one is exact in fp32, so both sides start from the same
    number; a draw's resolution is 2^-23."""
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def uniforms(seed: int, stream: int, request: int, position: int, count: int) -> np.ndarray:
    return to_uniform(words(seed, stream, request, position, count))


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variate -ln(-ln u)."""
    return -np.log(-np.log(u))
