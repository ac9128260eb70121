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


# ---------------------------------------------------------------------------
# Data-dependent filters (summary page, "Datenabhaengige Filter-Erweiterung
# (Appendix B)": a modified tiling, Algorithm 5, supports a filter that
# depends on the data at twice the work; the rebuttal adds that each step then
# runs two transforms of the same size instead of one).  The pages give no
# more detail.  Reading adopted: both sequences arrive online, x_n and the tap
# h_n at step n (0-based), and y_n = sum_{i+j=n} x_i h_j.  The pairs (i, j)
# are split once each into
#   red cells   (n, 0) and (0, n)                       at step n,
#   squares     x[p, 2p) x h[p, 2p)                      at step 2p - 1,
#   band blocks x[mp, (m+1)p) x h[p, 2p) and
#               h[mp, (m+1)p) x x[p, 2p), m >= 2         at step (m+1)p - 1,
# p a power of two: (i, j) with 1 <= j <= i lies in the square or band block
# of p = 2^floor(log2 j), and symmetrically for j > i.  A block is formed as
# soon as its last input has arrived, and all its targets lie after that step.
# ---------------------------------------------------------------------------
def dd_blocks(n: int):
    """Blocks of step n (0-based): ``(kind, p, x_lo, h_lo)``, the product of
    x[x_lo, x_lo + p) and h[h_lo, h_lo + p) into targets x_lo + h_lo onward."""
    p = 1
    while (n + 1) % p == 0 and 2 * p <= n + 1:
        m = (n + 1) // p - 1
        if m == 1:
            yield "square", p, p, p
        else:
            yield "x", p, n + 1 - p, p
            yield "h", p, p, n + 1 - p
        p *= 2


def dd_red_pairs(n: int):
    """Pairs (i, j) added directly at step n: (0, 0) at n = 0, else (n, 0) and (0, n)."""
    return [(0, 0)] if n == 0 else [(n, 0), (0, n)]
