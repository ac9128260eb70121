"""The bench workload (18 layers, B=1, D=864, L=2^17, contracting filters
h ~ N(0,1) exp(-k/16384)/sqrt(L), tanh map and feedback) run exactly as the
bench times it -- default options with per-launch event timing, calibrated
split, chunks, no records -- and checked against the CPU oracle:

* free running: the last layer's output of 16 (b, c) chains against the fp64
  oracle over all 131072 positions (this stack contracts, so two correct
  evaluations stay within the tolerance over the whole run and the check needs
  no divergence horizon);
* the same generation with records on (the chunk kernel variant that also
  stores every layer's input and output) agrees with it bit for bit;
* the recorded run replays against the oracle, layer by layer, at the dyadic
  block boundaries where the gray blocks of every class write, and at random
  positions.

The fp64 oracle for the 16 chains runs in a thread (the C call releases the
interpreter) while the GPU works."""
import threading
import time

import numpy as np
import pytest
import torch

import oracle
from long_convolution_sequence_amd import fi, workloads
from tests._parity import TF_TOL, say

pytestmark = pytest.mark.gpu


def _boundaries(L, rng, k=300):
    """0-based output slots: 2^q - 1, 2^q, 2^q + 1 for every q, k*2^15 +- 1, and random ones."""
    pts = set()
    for q in range(L.bit_length()):
        for v in (2 ** q - 2, 2 ** q - 1, 2 ** q, 2 ** q + 1):
            if 0 <= v < L:
                pts.add(v)
    for j in range(1, L // 32768 + 1):
        for v in (j * 32768 - 1, j * 32768, j * 32768 + 1):
            if 0 <= v < L:
                pts.add(v)
    pts.update(rng.integers(0, L, k).tolist())
    return np.array(sorted(pts), dtype=np.int64)


@pytest.mark.timeout(900)
def test_bench_workload_free_running_full_length_and_records():
    w = workloads.WORKLOADS[4]
    say(f"case {w.name}: bench configuration, full length")
    t0 = time.time()
    h = workloads.filters(w)
    x1 = workloads.x_first(w)                                  # [B][D]
    say(f"  filters generated in {time.time() - t0:.1f}s")
    rng = np.random.default_rng(404)
    chains = np.sort(rng.choice(w.B * w.D, 16, replace=False))
    bs, cs = chains // w.D, chains % w.D
    ref = {}

    def run_oracle():
        t = time.time()
        ref["y"] = oracle.stack(h, cs.astype(np.int32), x1[bs, cs], w.L)[0][:, -1, :]   # [16][L]
        ref["s"] = time.time() - t

    th = threading.Thread(target=run_oracle)
    th.start()

    hdev = torch.from_numpy(h).cuda()
    xdev = torch.from_numpy(x1).cuda()
    # 1. exactly the bench's context and call
    with fi.Context(hdev, w.B, time_blocks=True) as ctx:
        paths = [p for (_, p, _, _) in ctx.tau_table()]
        split = next(q for q, p in enumerate(paths) if p == fi.PATH_FFT)
        ctx.set_input(xdev)
        torch.cuda.synchronize()
        t1 = time.time()
        y_bench = ctx.generate(w.L)
        torch.cuda.synchronize()
        say(f"  bench context: split {split}, {w.L} positions in {time.time() - t1:.3f}s")
        y_bench = y_bench.cpu().numpy()
    torch.cuda.empty_cache()
    # 2. records on, same split: the same arithmetic, bit for bit
    with fi.Context(hdev, w.B, record=True, tau_split=split) as ctx:
        assert [p for (_, p, _, _) in ctx.tau_table()] == paths
        ctx.set_input(xdev)
        y_rec = ctx.generate(w.L).cpu().numpy()
        assert np.array_equal(y_bench, y_rec), "records on/off differ"
        say("  records on/off: bit for bit equal over all positions")
        # 3. replay of the recorded run at the block boundaries
        ts = _boundaries(w.L, rng)
        worst = 0.0
        for l in (0, 9, 17):
            xs = ctx.history(l, 0).cpu().numpy()            # [L][B][D]
            ys = ctx.history(l, 1).cpu().numpy()
            for c in rng.choice(w.D, 6, replace=False):
                xrow = np.ascontiguousarray(xs[:, 0, c])
                r = oracle.conv_points(h[l, c], xrow, ts)
                tol = TF_TOL * np.abs(h[l, c].astype(np.float64)).sum() * np.abs(xrow).max()
                worst = max(worst, float(np.abs(ys[ts, 0, c] - r).max() / tol))
            del xs, ys
        say(f"  replay at {len(ts)} positions (layers 0, 9, 17): worst error/tolerance {worst:.3e}")
        assert worst <= 1.0
    del hdev
    torch.cuda.empty_cache()
    th.join()
    say(f"  oracle: 16 chains x {w.L} positions x {w.M} layers in {ref['s']:.1f}s")
    yr = ref["y"]
    gpu = y_bench[:, bs, cs].T                                 # [16][L]
    rel = float(np.abs(gpu - yr).max() / np.abs(yr).max())
    say(f"  free running over all {w.L} positions: max |y_gpu - y_ref| / max |y_ref| = {rel:.3e}")
    assert rel <= 1e-3
