"""GPU parity of gray blocks wider than one workgroup transform (split into
K sub-blocks with offset-tap spectra), against the CPU oracle at sampled
positions of full-length rows."""
import numpy as np
import pytest
import torch

import oracle
from long_convolution_sequence_amd import fi
from tests._parity import TF_TOL, say

pytestmark = pytest.mark.gpu


def _positions(L, rng, k=400):
    """Sampled 0-based output slots: the ends of every dyadic range plus random ones."""
    pts = set()
    for q in range(L.bit_length()):
        for v in (2 ** q - 1, 2 ** q, 2 ** q + 1):
            if 0 <= v < L:
                pts.add(v)
    pts.update(rng.integers(0, L, k).tolist())
    return np.array(sorted(pts), dtype=np.int64)


def _run_teacher_forced(M, B, D, L, vlog, seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((M, D, L)).astype(np.float32)
    h *= np.exp(-np.arange(L) / (L / 4.0)).astype(np.float32)
    x = rng.standard_normal((L, B, D)).astype(np.float32)
    with fi.Context(torch.from_numpy(h).cuda(), B, map=fi.MAP_IDENTITY, tau_mode=fi.TAU_FFT,
                    fft_max_log2=vlog) as ctx:
        y = ctx.prefill(torch.from_numpy(x).cuda()).cpu().numpy()
    ts = _positions(L, rng)
    worst = 0.0
    for b in range(B):
        for c in range(D):
            ref = oracle.conv_points(h[0, c], x[:, b, c], ts)
            tol = TF_TOL * np.abs(h[0, c].astype(np.float64)).sum() * np.abs(x[:, :, c]).max()
            worst = max(worst, np.abs(y[ts, b, c] - ref).max() / tol)
    return worst


def test_split_blocks_k2_k4_k8():
    M, B, D, L = 1, 2, 3, 65536
    say(f"case split blocks width 2^12 (K=2,4,8) M={M} B={B} D={D} L={L}")
    worst = _run_teacher_forced(M, B, D, L, 12, 21)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


def test_split_blocks_default_width_full_length():
    M, B, D, L = 1, 1, 2, 131072
    say(f"case split blocks width 2^14 (K=2,4) M={M} B={B} D={D} L={L}")
    worst = _run_teacher_forced(M, B, D, L, 14, 22)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
