"""The relaxed tiling, enumerated straight from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Flash Inference (arXiv 2410.12982), summary page, "Kachelung-Strategie
(Algorithmus 1)": for i = 1 .. L-1, U is the largest power of two dividing i;
the red cell adds y_i * rho_0 into z_i, and the gray block adds the
contribution of inputs [i-U+1, i] to outputs [i+1, i+U].  Position L gets its
red cell only (the loop returns z_i inside its body, so the last position's
output needs nothing after it).  Positions are 1-based as on the page.

Reading adopted where the page is silent: L is a power of two, so no tile runs
past L (Proposition 1's analysis assumes L = 2^P).
"""
from __future__ import annotations


def largest_pow2_dividing(i: int) -> int:
    """Largest power of two that divides i (i >= 1), by repeated doubling."""
    if i < 1:
        raise ValueError("position must be >= 1")
    u = 1
    while i % (2 * u) == 0:
        u *= 2
    return u


def gray_tiles(L: int):
    """Yield ``(i, U, (in_lo, in_hi), (out_lo, out_hi))`` for i = 1..L-1, 1-based inclusive."""
    for i in range(1, L):
        u = largest_pow2_dividing(i)
        yield i, u, (i - u + 1, i), (i + 1, i + u)


def red_cells(L: int):
    """Positions whose own-term y_i * rho_0 is added directly: i = 1..L."""
    return range(1, L + 1)
