"""GPU parity of the eager prefill (all positions of a layer at once: direct
sums inside blocks of G, batched FFT blocks above) against the oracle and
against P teacher-forced positions, through the C-ABI; then generation
continues from the state it leaves."""
import numpy as np
import pytest
import torch

from long_convolution_sequence_amd import fi, workloads
from tests._parity import check_replay, replay_ratio, say

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("P", [16, 48, 256, 496, 512])
def test_eager_prefill_matches_steps_and_oracle(P):
    M, B, D, L = 3, 2, 5, 1024
    say(f"case eager prefill M={M} B={B} D={D} L={L} P={P}")
    r = np.random.default_rng(31)
    h = (r.standard_normal((M, D, L)) * np.exp(-np.arange(L) / 128.0) * 0.2).astype(np.float32)
    x = r.standard_normal((P, B, D)).astype(np.float32)
    kw = dict(tau_split=4, record=True)            # G = 16 in both contexts
    with fi.Context(_cuda(h), B, **kw) as e, fi.Context(_cuda(h), B, eager_prefill=False, **kw) as s:
        ye = e.prefill(_cuda(x)).cpu().numpy()
        ys = s.prefill(_cuda(x)).cpu().numpy()
        assert e.position == s.position == P
        rel = np.abs(ye - ys).max() / np.abs(ys).max()
        worst = check_replay(h, e, count=P)
        say(f"  prefill: eager vs steps rel {rel:.2e}; replay worst error/tolerance {worst:.3e}")
        assert rel <= 1e-5
        assert worst <= 1.0
        # generation continues from the eager state: feedback to the end
        ge = e.generate(L - P).cpu().numpy()
        gs = s.generate(L - P).cpu().numpy()
        relg = np.abs(ge - gs).max() / np.abs(gs).max()
        worst = check_replay(h, e)
        say(f"  then generation: eager vs steps rel {relg:.2e}; replay worst error/tolerance {worst:.3e}")
        assert relg <= 1e-4
        assert worst <= 1.0


def test_eager_prefill_falls_back_where_it_does_not_apply():
    M, B, D, L = 2, 1, 3, 256
    r = np.random.default_rng(32)
    h = (r.standard_normal((M, D, L)) * 0.1).astype(np.float32)
    for P in (20, 255):                            # not a multiple of G; and G = 16 here
        x = r.standard_normal((P, B, D)).astype(np.float32)
        with fi.Context(_cuda(h), B, tau_split=4) as a, fi.Context(_cuda(h), B, tau_split=4,
                                                                  eager_prefill=False) as b:
            assert torch.equal(a.prefill(_cuda(x)), b.prefill(_cuda(x)))


def test_eager_prefill_long_prompts_wide_blocks():
    """Prompts past one workgroup transform (width 2^12 here): at P = L/2 the
    two-half blocks after n = 2^13 end inside the prompt (their prefill kernel)
    and the split block after n = P starts at the prompt's end (run after the
    layer loop with the generation kernels)."""
    M, B, D, L, P = 2, 2, 3, 32768, 16384
    say(f"case eager prefill wide blocks M={M} B={B} D={D} L={L} P={P} width 2^12")
    r = np.random.default_rng(34)
    h = (r.standard_normal((M, D, L)) * np.exp(-np.arange(L) / 4096.0) * 0.05).astype(np.float32)
    x = r.standard_normal((P, B, D)).astype(np.float32)
    kw = dict(tau_split=4, record=True, fft_max_log2=12)
    with fi.Context(_cuda(h), B, **kw) as e, fi.Context(_cuda(h), B, eager_prefill=False, **kw) as s:
        assert e.schedule(8192)[0] == 13 and e.schedule(16384)[0] == 14
        ye = e.prefill(_cuda(x)).cpu().numpy()
        ys = s.prefill(_cuda(x)).cpu().numpy()
        rel = np.abs(ye - ys).max() / np.abs(ys).max()
        worst = check_replay(h, e, count=P)
        say(f"  prefill: eager vs steps rel {rel:.2e}; replay worst error/tolerance {worst:.3e}")
        assert rel <= 1e-5
        assert worst <= 1.0
        ge = e.generate(L - P).cpu().numpy()
        gs = s.generate(L - P).cpu().numpy()
        relg = np.abs(ge - gs).max() / np.abs(gs).max()
        worst = check_replay(h, e)
        say(f"  then generation: eager vs steps rel {relg:.2e}; replay worst error/tolerance {worst:.3e}")
        assert relg <= 1e-4
        assert worst <= 1.0


@pytest.mark.parametrize("P", [16384, 32768, 65536])
def test_eager_prefill_full_size_workload(P):
    """18 layers, B=1, D=864, L=2^17 (the bench workload): P = 16384 (every
    block after n <= P one workgroup wide), 32768 (the two-half block after P)
    and 65536 (two-half blocks inside the prompt, the split block after P)."""
    w = workloads.WORKLOADS[4]
    say(f"case eager prefill {w.name} P={P}")
    h = workloads.filters(w)
    x = np.random.default_rng(33).standard_normal((P, w.B, w.D)).astype(np.float32)
    with fi.Context(_cuda(h), w.B, record=True) as e:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        ye = e.prefill(_cuda(x))
        t1.record()
        torch.cuda.synchronize()
        say(f"  eager prefill {t0.elapsed_time(t1):.2f} ms")
        ye = ye.cpu().numpy()
        worst = 0.0
        for l in (0, 9, 17):
            xs = e.history(l, 0, P).cpu().numpy()
            ys = e.history(l, 1, P).cpu().numpy()
            for c in (0, 431, 863):
                worst = max(worst, replay_ratio(h[l, c], xs[:, :, c].T, ys[:, :, c].T))
        say(f"  replay worst error/tolerance {worst:.3e}")
        assert worst <= 1.0
        gen = e.generate(4096).cpu().numpy()          # the schedule continues after the prompt
        assert np.isfinite(gen).all()
    with fi.Context(_cuda(h), w.B, eager_prefill=False) as s:
        ys = s.prefill(_cuda(x)).cpu().numpy()
        gs = s.generate(4096).cpu().numpy()
    rel = np.abs(ye - ys).max() / np.abs(ys).max()
    relg = np.abs(gen - gs).max() / np.abs(gs).max()
    say(f"  eager vs steps: prefill rel {rel:.2e}, next 4096 positions rel {relg:.2e}")
    assert rel <= 1e-5 and relg <= 1e-4
