"""GPU parity of the Hyena-style block mode (projection, gate, mixer, GELU MLP,
RMSNorm, tanh feedback) against the CPU oracle.

Checks, all on the GPU's own recorded values:
* per-layer convolution replay (mixer output vs the fp64 causal sum of the
  recorded convolution inputs), the teacher-forced tolerance;
* per-position block replay: the oracle recomputes q, v from the recorded
  layer input and the block output a from the recorded mixer output, in fp64;
* free-running feedback against the fp64 oracle up to half of the horizon
  where fp32 and fp64 evaluations of the same model still agree to 1e-3.
The block's internal reading (column order, no residual, RMSNorm eps) is not
fixed by the pages: "parity unpinned" beyond self-consistency.
"""
import numpy as np
import pytest
import torch

from long_convolution_sequence_amd import fi, workloads
from oracle import block as oblock
from tests._parity import check_replay, say

pytestmark = pytest.mark.gpu


def _weights(w):
    bits = workloads.hyena_weights(w)
    return bits, {k: workloads.bf16_bits_to_f32(v) for k, v in bits.items()}


def _block_replay(ctx, w, Wf, x1, positions):
    """Worst relative error of q (projection*gate) and a (block output) over positions."""
    worst_q = worst_a = 0.0
    for n in positions:                                          # 0-based position
        q = [ctx.history(l, 0, 1, n + 1).cpu().numpy()[0] for l in range(w.M)]
        c = [ctx.history(l, 1, 1, n + 1).cpu().numpy()[0] for l in range(w.M)]
        a = [ctx.history(l, 2, 1, n + 1).cpu().numpy()[0] for l in range(w.M)]
        prev = ctx.history(w.M - 1, 2, 1, n).cpu().numpy()[0] if n > 0 else None
        for l in range(w.M):
            if l > 0:
                xin = a[l - 1]
            elif n == 0:
                xin = x1
            else:
                xin = np.tanh(prev.astype(np.float64))
            qr, vr = oblock.project(xin, Wf["W"][l])
            worst_q = max(worst_q, np.abs(q[l] - qr).max() / max(np.abs(qr).max(), 1e-30))
            ar = oblock.finish(c[l], vr, Wf["W1"][l], Wf["W2"][l])
            worst_a = max(worst_a, np.abs(a[l] - ar).max() / max(np.abs(ar).max(), 1e-30))
    return worst_q, worst_a


def _run(w, steps, prefix, replay_layers=None):
    bits, Wf = _weights(w)
    h = workloads.filters(w)
    x1 = workloads.x_first(w)
    with fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA, record=True) as ctx:
        ctx.set_block_weights(bits["W"], bits["W1"], bits["W2"])
        ctx.set_input(torch.from_numpy(x1).cuda())
        y = ctx.generate(steps).cpu().numpy()
        rng = np.random.default_rng(0)
        chans = None if w.D <= 64 else sorted(rng.choice(w.D, 8, replace=False))
        conv = check_replay(h, ctx, layers=replay_layers, chans=chans)
        pos = sorted(set([0, 1, 2, steps - 1] + [int(v) for v in rng.integers(0, steps, 6)]))
        wq, wa = _block_replay(ctx, w, Wf, x1, pos)
        a_last = ctx.history(w.M - 1, 2, prefix).cpu().numpy()
    assert np.array_equal(a_last, y[:prefix])        # y of fi_generate is a^{M-1}
    ref = oblock.generate(h, Wf["W"], Wf["W1"], Wf["W2"], x1, prefix)
    r32 = oblock.generate(h, Wf["W"], Wf["W1"], Wf["W2"], x1, prefix, dtype=np.float32)
    # Horizon: positions before two correct evaluations (fp32, fp64) drift apart by
    # 1e-4, a tenth of the tolerance.  The block's RMSNorm'd layers amplify rounding
    # strongly, so at full size even the first position can lie beyond it: then the
    # per-layer replay above carries parity and free-running adds nothing checkable.
    scale = np.abs(ref["a"][:, -1]).max()
    d32 = np.abs(r32["a"][:, -1] - ref["a"][:, -1]).reshape(prefix, -1).max(axis=1) / scale
    over = np.nonzero(d32 > 1e-4)[0]
    horizon = int(over[0]) if over.size else prefix
    dg = np.abs(y[:prefix] - ref["a"][:, -1]).reshape(prefix, -1).max(axis=1) / scale
    rel = float(dg[:horizon].max()) if horizon > 0 else 0.0
    return conv, wq, wa, horizon, rel, float(d32[0])


def test_block_mode_small():
    w = workloads.custom(M=2, B=2, D=64, L=256, decay=32.0, seed=31, block="hyena",
                         name="hyena M=2 B=2 D=64 L=2^8")
    say(f"case {w.name}")
    conv, wq, wa, horizon, rel, d0 = _run(w, w.L, 64)
    say(f"  conv replay {conv:.2e}; block replay q {wq:.2e} a {wa:.2e}; "
        f"horizon {horizon}, free-running {rel:.2e}")
    assert conv <= 1.0
    assert wq <= 1e-4 and wa <= 1e-4
    assert horizon >= 8 and rel <= 1e-3


def test_block_mode_full_size():
    """18 layers, B=4, D=768, L=2^15 Hyena-style block workload."""
    w = workloads.WORKLOADS[5]
    say(f"case {w.name}")
    conv, wq, wa, horizon, rel, d0 = _run(w, w.L, 16, replay_layers=(0, 17))
    say(f"  conv replay {conv:.2e}; block replay q {wq:.2e} a {wa:.2e}; horizon {horizon} "
        f"(fp32 vs fp64 oracle at the first position: {d0:.1e}), free-running {rel:.2e}")
    assert conv <= 1.0
    assert wq <= 1e-4 and wa <= 1e-4
    assert rel <= 1e-3


def test_block_kernel_timing_needs_reset():
    """fi_time_hyena_block times one position's block kernels and leaves the
    context needing a reset, like the other timing calls."""
    w = workloads.custom(M=2, B=2, D=32, L=64, decay=16.0, seed=71, block="hyena")
    say(f"case block kernel timing {w.name}")
    bits, _ = _weights(w)
    h = workloads.filters(w)
    with fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA) as ctx:
        with pytest.raises(fi.FiError) as e:
            ctx.time_hyena_block(3)                  # no weights yet
        assert e.value.status == fi.FI_ESTATE
    with fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA) as ctx:
        ctx.set_block_weights(bits["W"], bits["W1"], bits["W2"])
        us = ctx.time_hyena_block(5)
        assert 0.0 < us < 1e5
        with pytest.raises(fi.FiError) as e:
            ctx.step()
        assert e.value.status == fi.FI_ESTATE
        ctx.reset()
        ctx.set_input(torch.from_numpy(workloads.x_first(w)).cuda())
        ctx.generate(w.L, want_y=False)
        assert ctx.position == w.L
