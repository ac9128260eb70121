"""Algorithm 1 evaluated tile by tile in fp64 (teacher forcing).

TEST INFRASTRUCTURE ONLY, and a pin aid rather than the oracle proper: the
oracle's answer is the plain definition in ``naive.c``.  This module exists to
show, on the CPU and independently of the GPU code, that the reading of the
tiling (which inputs, which outputs, which taps, where the red cell goes)
reproduces the definition exactly.

Flash Inference (arXiv 2410.12982), summary page:
* "Beitrags-Aggregations-Definition": tau(y, [l, r], rho, [l', r'])_t is the sum
  over i in [l, r] of y_i * rho_{t-i}, for t in [l', r'].
* "Kachelung-Strategie (Algorithmus 1)": per position i, the red cell then the
  gray block of edge U = largest power of two dividing i.
* Lemma 1 and "Zirkulaere Faltungs-Trick": the gray block can be computed with
  an FFT; a circular convolution of length 2U suffices because the wanted
  outputs (indices U .. 2U-1 of the circular result) are untouched by the
  wrap-around.
"""
from __future__ import annotations

import numpy as np

from .schedule import largest_pow2_dividing


def tau_direct(y, lo, hi, rho, out_lo, out_hi):
    """tau by its definition; 1-based inclusive ranges; y is indexed y[i-1]."""
    out = np.zeros(out_hi - out_lo + 1)
    for t in range(out_lo, out_hi + 1):
        acc = 0.0
        for i in range(lo, hi + 1):
            acc += y[i - 1] * rho[t - i]
        out[t - out_lo] = acc
    return out


def tau_circular_fft(y, i, U, rho):
    """The gray block after position i (inputs [i-U+1, i], outputs [i+1, i+U])
    as a length-2U circular convolution with taps rho[0..2U-1], keeping the
    circular outputs at indices U..2U-1."""
    a = np.zeros(2 * U)
    a[:U] = y[i - U:i]            # y_{i-U+1} .. y_i  (1-based)
    g = np.asarray(rho[:2 * U], dtype=np.float64)
    c = np.fft.ifft(np.fft.fft(a) * np.fft.fft(g)).real
    return c[U:2 * U]


def relaxed_conv(rho, y, tile="direct"):
    """z_t = sum_{i<=t} y_i rho_{t-i} for t = 1..L, computed by Algorithm 1.

    ``tile`` selects the gray-block evaluation: "direct" (tau by definition)
    or "fft" (circular 2U trick).  Returns fp64 z[0..L-1] (z_t at index t-1).
    """
    y = np.asarray(y, dtype=np.float64)
    rho = np.asarray(rho, dtype=np.float64)
    L = y.shape[0]
    z = np.zeros(L + 1)              # 1-based accumulators, z[0] unused
    out = np.zeros(L)
    for i in range(1, L + 1):
        z[i] += y[i - 1] * rho[0]    # red cell
        out[i - 1] = z[i]            # z_i is final and returned here
        if i == L:
            break
        U = largest_pow2_dividing(i)
        if tile == "direct":
            blk = tau_direct(y, i - U + 1, i, rho, i + 1, i + U)
        elif tile == "fft":
            blk = tau_circular_fft(y, i, U, rho)
        else:
            raise ValueError(tile)
        z[i + 1:i + U + 1] += blk     # gray block
    return out
