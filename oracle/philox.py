"""Philox4x32-10 counter-based generator, in plain Python integers.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11. A 4-word counter and a 2-word key; each round
multiplies words 0 and 2 by fixed odd constants, keeps both halves of the 64-bit
products, and mixes the high halves with words 1 and 3 and the key. Between rounds
the key is advanced by the two Weyl constants (the golden ratio and sqrt(3) - 1,
scaled to 32 bits). Ten rounds.

Stochastic rounding ([WB] "Post-training write-back interventions and diagnostics";
[WB-zh] "Error feedback and stochastic rounding" 误差反馈与随机舍入) only needs an
unbiased uniform draw per element. The pages fix no generator; the draw used here,
and by the GPU independently, is one 16-bit slice of a Philox output:
    key     = (seed mod 2^32, seed >> 32)
    counter = (16*row + col // 8, b*H + h, t mod 2^32, t >> 32)
    element col uses output word (col mod 8) // 2, its low half when col is even,
    its high half when col is odd.
Parity of this mapping is unpinned beyond the agreement of two implementations; the
generator itself is pinned by the published known-answer vectors (tests).
"""
from __future__ import annotations

MASK32 = 0xFFFFFFFF
MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85


def philox4x32_10(counter, key):
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
        p0 = MUL0 * c0
        p1 = MUL1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK32, lo1, (hi0 ^ c3 ^ k1) & MASK32, lo0
    return (c0, c1, c2, c3)


def sr_draws(seed: int, b: int, h: int, H: int, t: int, row: int, ncols: int):
    """16-bit uniform draws for the ``ncols`` elements of one stored row."""
    key = (seed & MASK32, (seed >> 32) & MASK32)
    out = []
    for col in range(ncols):
        if col % 8 == 0:
            words = philox4x32_10((16 * row + col // 8, b * H + h, t & MASK32,
                                   (t >> 32) & MASK32), key)
        w = words[(col % 8) // 2]
        out.append(w & 0xFFFF if col % 2 == 0 else w >> 16)
    return out
