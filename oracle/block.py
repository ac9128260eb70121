"""Hyena-style block of the 18-layer, B=4, D=768, L=2^15 block workload, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Flash Inference (arXiv 2410.12982), summary page, "Modellarchitektur": each
layer is a position mixer (the long convolution) followed by a per-position
block R^D -> R^D; "Experimentelle Einrichtung" names Hyena and blocks made of
an MLP with GELU.  The pages do not spell out Hyena's internals, so this
oracle takes the plainest reading of the workload's own outline (all choices
are listed with the tests; "parity unpinned" where no page fixes them):

* ``[u | v | w] = x W`` with W of shape (D, 3D): columns [0, D), [D, 2D), [2D, 3D);
* the convolution input is ``q = u * w`` (elementwise);
* the mixer output at position t is ``c_t = sum_{s<=t} h_{t-s} q_s``;
* ``m = v * c``; MLP ``W2 GELU(W1 m)`` with W1 (D, 4D), W2 (4D, D), no biases,
  GELU with the exact normal CDF ``z * Phi(z)``;
* ``a = RMSNorm(MLP)`` = ``z / sqrt(mean(z^2) + 1e-6)`` with unit gain, no residual;
* the next layer's input is a; the next position's layer-0 input is tanh(a^{M-1}).

Row vectors: x has shape (B, D) and multiplies weights from the left.  The
weights are given as bf16 values already widened to float; arithmetic is fp64.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

RMS_EPS = 1e-6


def gelu(z):
    """z * Phi(z) with Phi the standard normal CDF, via erf (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def rmsnorm(z, eps=RMS_EPS):
    """z / sqrt(mean(z^2 over the last axis) + eps), unit gain (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def project(x, W):
    """Return (q, v): q = u*w is the convolution input, v gates its output."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    D = x.shape[-1]
    uvw = x @ W
    u, v, w = uvw[..., :D], uvw[..., D:2 * D], uvw[..., 2 * D:3 * D]
    return u * w, v


def finish(c, v, W1, W2):
    """Given the mixer output c and gate v: a = RMSNorm(W2 GELU(W1 (v*c)))."""
    m = np.asarray(v, dtype=np.float64) * np.asarray(c, dtype=np.float64)
    hidden = gelu(m @ np.asarray(W1, dtype=np.float64))
    return rmsnorm(hidden @ np.asarray(W2, dtype=np.float64))


def generate(filters, W, W1, W2, x_first, steps, dtype=np.float64):
    """Whole-model feedback generation for ``steps`` positions.

    filters : [M, D, L]; W, W1, W2 : [M, ...] per-layer weights (float arrays);
    x_first : [B, D] layer-0 input at the first position.
    Returns dict with arrays q, c, a of shape [steps, M, B, D].
    dtype fp64 is the oracle; fp32 (same operations, rounded to fp32 after each
    step) exists only to measure how fast two correct evaluations diverge.
    Cost is O(steps^2 * M * B * D) for the convolutions: small cases only.
    """
    f64 = dtype == np.float64

    def r(a):
        return np.asarray(a, dtype=np.float64) if f64 else np.asarray(a, dtype=np.float32).astype(np.float64)

    filters = np.asarray(filters, dtype=np.float64)
    M, D, L = filters.shape
    B = x_first.shape[0]
    q_hist = np.zeros((M, steps, B, D))
    Q = np.zeros((steps, M, B, D))
    C = np.zeros((steps, M, B, D))
    A = np.zeros((steps, M, B, D))
    x = r(x_first)
    for n in range(steps):
        for l in range(M):
            q, v = project(x, W[l])
            q, v = r(q), r(v)
            q_hist[l, n] = q
            # c_n[b, ch] = sum_{s<=n} h^l[ch][n-s] q_s[b, ch]
            taps = filters[l, :, n::-1]                  # [D, n+1]: h[n-s] for s = 0..n
            c = r(np.einsum("sbd,ds->bd", q_hist[l, :n + 1], taps))
            a = r(finish(c, v, W1[l], W2[l]))
            Q[n, l], C[n, l], A[n, l] = q, c, a
            x = a
        x = r(np.tanh(A[n, M - 1]))
    return {"q": Q, "c": C, "a": A}
