"""Data-dependent filters (fi_dd_*): parity with the definition y_t = sum_{i+j=t} x_i h_j.

Flash Inference (arXiv 2410.12982), summary page, "Datenabhaengige Filter-Erweiterung
(Appendix B)": the taps depend on the data, so they arrive online with the inputs; the oracle
is the plain causal convolution of the realised sequences (oracle.conv_rows, fp64), and the
tolerance is the teacher-forced bar 1e-4 * ||h||_1 * max|x| per row.
"""
import numpy as np
import pytest
import torch

import oracle
from long_convolution_sequence_amd import fi
from tests._parity import TF_TOL, say

pytestmark = pytest.mark.gpu


def _rows_worst(x, h, y):
    """x, h, y: [T][B][D]; worst error / tolerance over all rows against the oracle."""
    T = x.shape[0]
    xr = np.ascontiguousarray(x.reshape(T, -1).T)
    hr = np.ascontiguousarray(h.reshape(T, -1).T)
    ref = oracle.conv_rows(hr, xr)
    got = y.reshape(T, -1).T
    worst = 0.0
    for r in range(xr.shape[0]):
        tol = TF_TOL * np.abs(hr[r].astype(np.float64)).sum() * np.abs(xr[r]).max()
        worst = max(worst, np.abs(got[r] - ref[r]).max() / tol)
    return worst


def _seq(T, B, D, seed, decay):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, B, D)).astype(np.float32)
    h = (rng.standard_normal((T, B, D)) * np.exp(-np.arange(T) / decay)[:, None, None]).astype(np.float32)
    return x, h


@pytest.mark.parametrize("fft_min", [2, 3, 5, 7, 8, 15])
def test_dd_matches_definition(fft_min):
    B, D, L = 2, 5, 1024
    say(f"case data-dependent B={B} D={D} L={L} fft_min_log2={fft_min}")
    x, h = _seq(L, B, D, 41, 300.0)
    with fi.DDContext(B, D, L, fft_min_log2=fft_min) as ctx:
        y = ctx.run(torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
        assert ctx.position == L
        with pytest.raises(fi.FiError):
            ctx.step(torch.from_numpy(x[0]).cuda(), torch.from_numpy(h[0]).cuda())
    worst = _rows_worst(x, h, y)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


def test_dd_steps_equal_run_and_reset_repeats():
    B, D, L = 1, 7, 256
    say(f"case data-dependent steps/run/reset B={B} D={D} L={L}")
    x, h = _seq(L, B, D, 42, 100.0)
    xd, hd = torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()
    with fi.DDContext(B, D, L, fft_min_log2=3) as ctx:
        ys = torch.stack([ctx.step(xd[t], hd[t]) for t in range(L)]).cpu().numpy()
        ctx.reset()
        assert ctx.position == 0
        yr = ctx.run(xd, hd).cpu().numpy()
    assert np.array_equal(ys, yr)


def test_dd_taps_made_from_the_outputs():
    """Both sequences depend on the outputs so far (x_{t+1} = tanh(y_t) + noise,
    h_{t+1} = 0.3 tanh(y_t) e^{-t/150}), so each arrives only after the previous position: the
    realised sequences, recorded, are checked against the definition."""
    B, D, L = 2, 3, 512
    say(f"case data-dependent taps from outputs B={B} D={D} L={L}")
    rng = np.random.default_rng(43)
    noise = torch.from_numpy(rng.standard_normal((L, B, D)).astype(np.float32) * 0.1).cuda()
    xs = torch.empty((L, B, D), device="cuda")
    hs = torch.empty((L, B, D), device="cuda")
    ys = torch.empty((L, B, D), device="cuda")
    xs[0] = torch.from_numpy(rng.standard_normal((B, D)).astype(np.float32)).cuda()
    hs[0] = 1.0
    with fi.DDContext(B, D, L, fft_min_log2=4) as ctx:
        for t in range(L):
            ctx.step(xs[t], hs[t], ys[t])
            if t + 1 < L:
                xs[t + 1] = torch.tanh(ys[t]) + noise[t]
                hs[t + 1] = 0.3 * torch.tanh(ys[t]) * float(np.exp(-t / 150.0))
    worst = _rows_worst(xs.cpu().numpy(), hs.cpu().numpy(), ys.cpu().numpy())
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


def test_dd_widest_products_sampled_rows():
    """L = 2^15, the widest products (p = 2^14) one workgroup's transform; 6 of 256 rows checked."""
    B, D, L = 1, 256, 32768
    say(f"case data-dependent full width B={B} D={D} L={L}")
    x, h = _seq(L, B, D, 44, 4096.0)
    with fi.DDContext(B, D, L) as ctx:
        y = ctx.run(torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
    rows = [0, 17, 100, 128, 201, 255]
    worst = _rows_worst(x[:, :, rows], h[:, :, rows], y[:, :, rows])
    say(f"  worst error/tolerance over {len(rows)} rows {worst:.3e}")
    assert worst <= 1.0


@pytest.mark.parametrize("L", [1, 2, 4, 8, 16])
def test_dd_tiny_lengths(L):
    """The degenerate lengths: red cells only (L <= 2), one square (L = 4), the
    first band products (L = 8, 16)."""
    B, D = 1, 3
    say(f"case data-dependent tiny B={B} D={D} L={L}")
    x, h = _seq(L, B, D, 45 + L, 4.0)
    with fi.DDContext(B, D, L) as ctx:
        y = ctx.run(torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
        assert ctx.position == L
    assert _rows_worst(x, h, y) <= 1.0


def test_dd_many_rows_ragged():
    """B*D = 1011 rows: several blocks of the per-row kernels and a partly
    filled last one."""
    B, D, L = 3, 337, 2048
    say(f"case data-dependent rows B={B} D={D} L={L}")
    x, h = _seq(L, B, D, 46, 500.0)
    with fi.DDContext(B, D, L) as ctx:
        y = ctx.run(torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
    worst = _rows_worst(x, h, y)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


@pytest.mark.parametrize("fft_min", [3, 8])
def test_dd_stack_layers_replayed_against_definition(fft_min):
    """A stack of data-dependent layers (fi_dd_stack_*): layer 0's input and every
    layer's taps arrive per position, layer l+1's input is tanh(y^l_t).  Each layer
    is replayed against the definition from its realised input (layer 0: the given
    one; layer l+1: tanh of the GPU's layer-l output, in fp32), so every layer meets
    the teacher-forced bar; steps and run agree bit for bit, reset repeats."""
    M, B, D, L = 3, 2, 5, 4096
    say(f"case data-dependent stack M={M} B={B} D={D} L={L} fft_min_log2={fft_min}")
    rng = np.random.default_rng(43)
    x0 = rng.standard_normal((L, B, D)).astype(np.float32)
    h = (rng.standard_normal((L, M, B, D)) * np.exp(-np.arange(L) / 600.0)[:, None, None, None]
         / np.sqrt(60.0)).astype(np.float32)
    xd, hd = torch.from_numpy(x0).cuda(), torch.from_numpy(h).cuda()
    with fi.DDContext(B, D, L, fft_min_log2=fft_min, layers=M) as ctx:
        y = ctx.run(xd, hd).cpu().numpy()                       # [L][M][B][D]
        assert ctx.position == L
        ctx.reset()
        half = L // 2
        ya = torch.stack([ctx.step(xd[t], hd[t]) for t in range(100)])
        yb = ctx.run(xd[100:half], hd[100:half])
        yc = ctx.run(xd[half:], hd[half:])
        assert np.array_equal(torch.cat([ya, yb, yc]).cpu().numpy(), y)
    worst = 0.0
    xl = x0
    for l in range(M):
        w = _rows_worst(xl, np.ascontiguousarray(h[:, l]), np.ascontiguousarray(y[:, l]))
        say(f"  layer {l}: worst error/tolerance {w:.3e}, max|y| {np.abs(y[:, l]).max():.3f}")
        worst = max(worst, w)
        xl = np.tanh(y[:, l]).astype(np.float32)
    assert worst <= 1.0
    assert np.abs(y[:, M - 1]).max() > 1e-3


def test_dd_stack_of_one_layer_equals_single_layer():
    """layers=1 runs the stack path (the red-cell kernel, then the products); it must
    give the single-layer context's outputs bit for bit."""
    B, D, L = 2, 3, 1024
    say(f"case data-dependent stack of one layer B={B} D={D} L={L}")
    x, h = _seq(L, B, D, 44, 200.0)
    xd, hd = torch.from_numpy(x).cuda(), torch.from_numpy(h).cuda()
    with fi.DDContext(B, D, L, fft_min_log2=5) as one:
        y1 = one.run(xd, hd).cpu().numpy()
    with fi.DDContext(B, D, L, fft_min_log2=5, layers=1) as st:
        ys = st.run(xd, hd[:, None]).cpu().numpy()
    assert np.array_equal(ys[:, 0], y1)
