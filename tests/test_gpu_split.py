"""GPU parity of gray blocks wider than one workgroup transform: the class of
twice that width (two halves in one workgroup) and the wider classes (split
into K sub-blocks with offset-tap spectra), against the CPU oracle at sampled
positions of full-length rows; and the deferred later sub-blocks of split
blocks (defer_wide): the deferred run replays against the oracle and equals
the undeferred run bit for bit."""
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
    say(f"case two-half block 2^13, split blocks 2^14, 2^15 (K=4, 8) M={M} B={B} D={D} L={L}")
    worst = _run_teacher_forced(M, B, D, L, 12, 21)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


def test_split_blocks_default_width_full_length():
    M, B, D, L = 1, 1, 2, 131072
    say(f"case two-half block 2^15, split block 2^16 (K=4) M={M} B={B} D={D} L={L}")
    worst = _run_teacher_forced(M, B, D, L, 14, 22)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


def test_split_blocks_k16_full_length():
    """Width 2^12 at L = 2^17: split blocks with K = 4, 8 and 16 sub-blocks
    (K = 16 takes the kernel whose sub-block count is not fixed at compile time)."""
    M, B, D, L = 1, 1, 2, 131072
    say(f"case two-half block 2^13, split blocks 2^14, 2^15, 2^16 (K=4, 8, 16) M={M} B={B} D={D} L={L}")
    worst = _run_teacher_forced(M, B, D, L, 12, 23)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


@pytest.mark.parametrize("graphs", [True, False])
def test_deferred_split_sub_blocks_change_nothing(graphs):
    """Feedback stack with split classes 2^14 and 2^15 (width 2^12): generation
    and single steps with the later sub-blocks deferred to the side stream equal
    the undeferred run bit for bit, also when a run stops inside a deferral."""
    M, B, D, L = 2, 2, 5, 32768
    say(f"case deferred split sub-blocks M={M} B={B} D={D} L={L} graphs={graphs}")
    rng = np.random.default_rng(31)
    h = (rng.standard_normal((M, D, L)) * np.exp(-np.arange(L) / 4096.0) / np.sqrt(L)).astype(np.float32)
    x1 = torch.from_numpy(rng.standard_normal((B, D)).astype(np.float32)).cuda()
    outs = []
    worst = 0.0
    for defer in (False, True):
        with fi.Context(torch.from_numpy(h).cuda(), B, tau_split=6, fft_max_log2=12, use_graphs=graphs,
                        defer_wide=defer, record=defer) as ctx:
            ctx.set_input(x1)
            a = ctx.generate(16384 + 100)          # stops 100 positions into the first deferral
            b = torch.stack([ctx.step() for _ in range(200)])
            c = ctx.generate(L - 16384 - 300)
            outs.append(torch.cat([a, b, c]).cpu().numpy())
            if defer:
                # the deferred run itself against the oracle: every layer, every (b, c), replayed
                # from its recorded inputs at the ends of every dyadic range (where the split
                # classes' output sub-blocks start and end) and at random positions
                ts = _positions(L, rng, 200)
                ts = np.unique(np.concatenate([ts, np.arange(16384, L, 4096) - 1, np.arange(16384, L, 4096)]))
                for l in range(M):
                    xs = ctx.history(l, 0).cpu().numpy()
                    ys = ctx.history(l, 1).cpu().numpy()
                    for bb in range(B):
                        for cc in range(D):
                            xrow = np.ascontiguousarray(xs[:, bb, cc])
                            ref = oracle.conv_points(h[l, cc], xrow, ts)
                            tol = TF_TOL * np.abs(h[l, cc].astype(np.float64)).sum() * np.abs(xrow).max()
                            worst = max(worst, float(np.abs(ys[ts, bb, cc] - ref).max() / tol))
    say(f"  deferred run vs oracle (replay at {len(ts)} positions): worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
    assert np.array_equal(outs[0], outs[1])
    assert np.abs(outs[0]).max() > 0


@pytest.mark.parametrize("graphs", [True, False])
def test_deferred_two_half_blocks_against_oracle(graphs):
    """defer_wide = 2 with width 2^13 at L = 2^16: the two-half class 2^14 runs
    as 4 sub-blocks of 2^12 with sub-blocks 1..3 on the side stream, the split
    class 2^15 as with level 1.  Every layer of the free-running stack is
    replayed from its recorded inputs against the oracle (at the ends of every
    dyadic range, the sub-block boundaries after each wide block, and random
    positions), also when a run stops inside a deferral; graphs on and off give
    the same outputs; a context made without level 2 refuses it."""
    M, B, D, L = 2, 2, 5, 65536
    say(f"case deferred two-half blocks M={M} B={B} D={D} L={L} graphs={graphs}")
    rng = np.random.default_rng(37)
    h = (rng.standard_normal((M, D, L)) * np.exp(-np.arange(L) / 8192.0) / np.sqrt(L)).astype(np.float32)
    x1 = torch.from_numpy(rng.standard_normal((B, D)).astype(np.float32)).cuda()
    with fi.Context(torch.from_numpy(h).cuda(), B, tau_split=6, fft_max_log2=13, use_graphs=graphs,
                    defer_wide=1) as ctx:
        with pytest.raises(fi.FiError):
            ctx.set_defer_wide(2)
    with fi.Context(torch.from_numpy(h).cuda(), B, tau_split=6, fft_max_log2=13, use_graphs=graphs,
                    defer_wide=2, record=True) as ctx:
        ctx.set_input(x1)
        a = ctx.generate(16384 + 100)              # stops 100 positions into the first two-half deferral
        b = torch.stack([ctx.step() for _ in range(200)])
        c = ctx.generate(49152 - 16384 - 300)      # up to the second two-half block
        d = ctx.generate(L - 49152)
        y = torch.cat([a, b, c, d]).cpu().numpy()
        ts = _positions(L, rng, 200)
        ends = np.concatenate([np.arange(16384, 16384 + 16384 + 1, 4096), np.arange(49152, L + 1, 4096),
                               np.arange(32768, L + 1, 8192)])
        ts = np.unique(np.concatenate([ts, ends - 1, ends[ends < L]]))
        worst = 0.0
        for l in range(M):
            xs = ctx.history(l, 0).cpu().numpy()
            ys = ctx.history(l, 1).cpu().numpy()
            for bb in range(B):
                for cc in range(D):
                    xrow = np.ascontiguousarray(xs[:, bb, cc])
                    ref = oracle.conv_points(h[l, cc], xrow, ts)
                    tol = TF_TOL * np.abs(h[l, cc].astype(np.float64)).sum() * np.abs(xrow).max()
                    worst = max(worst, float(np.abs(ys[ts, bb, cc] - ref).max() / tol))
    say(f"  level-2 deferred run vs oracle (replay at {len(ts)} positions): worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
    assert np.abs(y).max() > 0
    assert np.isfinite(y).all()
