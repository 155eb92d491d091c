"""SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), written from its published definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The block pool shuffles its initial free list with this generator so that the
physical placement of blocks is scattered but reproducible.  The library's C++
pool implements the same published generator on its own; neither side calls
the other.

Definition: the state advances by the odd constant 0x9E3779B97F4A7C15 (the
64-bit golden ratio); the output is the state passed through the variant-13
64-bit finaliser: xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift 27,
multiply 0x94D049BB133111EB, xor-shift 31, all modulo 2^64.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1


class SplitMix64:
    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def shuffled_order(n: int, seed: int) -> list[int]:
    """Fisher-Yates (Durstenfeld) shuffle of [0, n): for i = n-1 down to 1,
    j = next() mod (i+1), swap a[i], a[j].  Seed 0 means no shuffle."""
    a = list(range(n))
    if seed == 0:
        return a
    g = SplitMix64(seed)
    for i in range(n - 1, 0, -1):
        j = g.next() % (i + 1)
        a[i], a[j] = a[j], a[i]
    return a
