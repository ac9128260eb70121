"""GPU parity of the relaxed-tiling HIP path against the CPU oracle, through
the C-ABI (ctypes binding).  Small shapes that still span every block-size
class, both block paths and ragged chain counts."""
import numpy as np
import pytest
import torch

import oracle
from long_convolution_sequence_amd import fi, workloads
from tests._parity import TF_TOL, check_replay, say

pytestmark = pytest.mark.gpu

TAUS = {"direct": fi.TAU_DIRECT, "fft": fi.TAU_FFT, "auto": fi.TAU_AUTO}


def _filters(M, D, L, seed, decay=None):
    r = np.random.default_rng(seed)
    h = r.standard_normal((M, D, L))
    if decay:
        h *= np.exp(-np.arange(L) / decay)
    return h.astype(np.float32)


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("tau", list(TAUS))
def test_single_layer_teacher_forced_matches_definition(tau):
    M, B, D, L = 1, 2, 5, 256
    say(f"case single-layer teacher-forced tau={tau} M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 1)
    x = np.random.default_rng(2).standard_normal((L, B, D)).astype(np.float32)
    with fi.Context(_cuda(h), B, tau_mode=TAUS[tau], map=fi.MAP_IDENTITY) as ctx:
        paths = [p for (_, p, _, _) in ctx.tau_table()]
        if tau == "fft":
            assert all(p == fi.PATH_FFT for p in paths[2:]) and paths[:2] == [fi.PATH_DIRECT] * 2
        if tau == "direct":
            assert all(p == fi.PATH_DIRECT for p in paths)
        y = ctx.prefill(_cuda(x)).cpu().numpy()
        assert ctx.position == L
    worst = 0.0
    for b in range(B):
        for c in range(D):
            ref = oracle.conv_rows(h[0, c], x[:, b, c])
            tol = TF_TOL * np.abs(h[0, c].astype(np.float64)).sum() * np.abs(x[:, :, c]).max()
            worst = max(worst, np.abs(y[:, b, c] - ref).max() / tol)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
    # much tighter than the bar: the tiling adds only fp32 rounding
    assert worst <= 0.05


@pytest.mark.parametrize("chunk", [True, False])
@pytest.mark.parametrize("tau", list(TAUS))
def test_stack_teacher_forced_per_layer_replay(tau, chunk):
    M, B, D, L = 3, 2, 6, 512
    say(f"case stack teacher-forced replay tau={tau} chunk={chunk} M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 3, decay=128.0)
    x = np.random.default_rng(4).standard_normal((L, B, D)).astype(np.float32)
    with fi.Context(_cuda(h), B, tau_mode=TAUS[tau], record=True, chunk_direct=chunk) as ctx:
        y = ctx.prefill(_cuda(x)).cpu().numpy()
        x0 = ctx.history(0, 0).cpu().numpy()
        assert np.array_equal(x0, x)                                 # inputs land in their slots
        for l in range(M - 1):                                       # inter-layer map
            yl = ctx.history(l, 1).cpu().numpy()
            xn = ctx.history(l + 1, 0).cpu().numpy()
            assert np.allclose(xn, np.tanh(yl.astype(np.float64)), rtol=0, atol=4e-7)
        assert np.array_equal(ctx.history(M - 1, 1).cpu().numpy(), y)
        worst = check_replay(h, ctx)
    say(f"  worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


@pytest.mark.parametrize("chunk", [True, False])
def test_feedback_small_config_replay_and_horizon(chunk):
    """1 layer, B=1, D=4, L=1024, h ~ N(0,1) exp(-k/256), x_1 ~ N(0,1), x_{t+1} = tanh(y_t)."""
    w = workloads.WORKLOADS[1]
    say(f"case feedback {w.name} chunk={chunk}")
    h = workloads.filters(w)
    x1 = workloads.x_first(w)
    with fi.Context(_cuda(h), w.B, record=True, chunk_direct=chunk) as ctx:
        ctx.set_input(_cuda(x1))
        y = ctx.generate(w.L).cpu().numpy()            # [L][B][D]
        xs = ctx.history(0, 0).cpu().numpy()           # [L][B][D]
        worst = check_replay(h, ctx)
    say(f"  replay worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
    # the feedback wiring: x_1 given, x_{n+1} = tanh(y_n)
    assert np.array_equal(xs[0], x1)
    assert np.allclose(xs[1:], np.tanh(y[:-1].astype(np.float64)), rtol=0, atol=4e-7)
    # free-running against the fp64 oracle within the measured divergence horizon
    chans = np.arange(w.D)
    y64, _ = oracle.stack(h, chans, x1[0], w.L)
    y32, _ = oracle.stack_f32(h, chans, x1[0], w.L)
    scale = np.abs(y64[:, 0]).max()
    d32 = np.abs(y32[:, 0] - y64[:, 0]).max(axis=0) / scale
    over = np.nonzero(d32 > 1e-3)[0]
    horizon = int(over[0]) if over.size else w.L
    dgpu = np.abs(y[:, 0, :].T - y64[:, 0]).max(axis=0) / scale
    say(f"  fp32-vs-fp64 horizon {horizon}; GPU rel error over first half {dgpu[:horizon // 2].max():.2e}")
    assert horizon >= 256
    assert dgpu[:horizon // 2].max() <= 1e-3


@pytest.mark.parametrize("chunk", [True, False])
def test_paths_agree_and_runs_are_deterministic(chunk):
    M, B, D, L = 2, 3, 7, 1024
    say(f"case path agreement chunk={chunk} M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 5, decay=300.0) * 0.05
    x1 = np.random.default_rng(6).standard_normal((B, D)).astype(np.float32)
    outs, paths = {}, {}
    for name, tau in TAUS.items():
        split = -1
        for graphs in (True, False):
            # "auto" calibrates in the first context; the second takes the split it chose (a second
            # calibration could pick another, and with it another order of the additions)
            with fi.Context(_cuda(h), B, tau_mode=tau, tau_split=split, use_graphs=graphs,
                            chunk_direct=chunk) as ctx:
                paths[(name, graphs)] = [q[1] for q in ctx.tau_table()]
                if name == "auto":
                    split = next((q for q, p in enumerate(paths[(name, graphs)]) if p == fi.PATH_FFT), ctx.P)
                ctx.set_input(_cuda(x1))
                outs[(name, graphs)] = ctx.generate(L).cpu().numpy()
    for name in TAUS:
        assert paths[(name, True)] == paths[(name, False)], name
        assert np.array_equal(outs[(name, True)], outs[(name, False)]), name
    ref = outs[("direct", True)]
    for name in ("fft", "auto"):
        rel = np.abs(outs[(name, True)] - ref).max() / np.abs(ref).max()
        say(f"  {name} vs direct rel diff {rel:.2e}")
        assert rel <= 1e-3
    with fi.Context(_cuda(h), B, tau_mode=fi.TAU_FFT, chunk_direct=chunk) as ctx:
        ctx.set_input(_cuda(x1))
        again = ctx.generate(L).cpu().numpy()
    assert np.array_equal(again, outs[("fft", True)])


def test_prefill_equals_steps_then_generation_continues():
    M, B, D, L, P = 2, 2, 5, 256, 77
    say(f"case prefill == steps M={M} B={B} D={D} L={L} P={P}")
    h = _filters(M, D, L, 7, decay=64.0)
    x = np.random.default_rng(8).standard_normal((P, B, D)).astype(np.float32)
    # one fixed split for both contexts: two calibrations may pick different
    # paths, which agree only to rounding; one launch per position in both
    with fi.Context(_cuda(h), B, tau_split=4, chunk_direct=False) as a, \
            fi.Context(_cuda(h), B, tau_split=4, chunk_direct=False) as b:
        ya = a.prefill(_cuda(x))
        yb = torch.stack([b.step(_cuda(x[i])) for i in range(P)])
        assert torch.equal(ya, yb)
        ga = a.generate(L - P)
        gb = torch.cat([b.step()[None] for _ in range(L - P)])
        assert torch.equal(ga, gb)
        assert a.position == b.position == L
        with pytest.raises(fi.FiError) as e:
            a.step()
        assert e.value.status == fi.FI_ERANGE


def test_lazy_baseline_matches_tiled():
    M, B, D, L = 2, 2, 3, 256
    say(f"case lazy vs tiled M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 9, decay=64.0) * 0.2
    x1 = np.random.default_rng(10).standard_normal((B, D)).astype(np.float32)
    with fi.Context(_cuda(h), B, record=True) as ctx:
        ctx.set_input(_cuda(x1))
        yt = ctx.generate(L).cpu().numpy()
        ctx.reset()
        ctx.set_input(_cuda(x1))
        yl = ctx.lazy_generate(L).cpu().numpy()
        worst = check_replay(h, ctx)
        ctx.reset()
        ctx.lazy_generate(10, want_y=False)
        with pytest.raises(fi.FiError) as e:       # tiled and Lazy state do not mix
            ctx.generate(1)
        assert e.value.status == fi.FI_ESTATE
    say(f"  lazy replay worst {worst:.2e}; lazy vs tiled {np.abs(yl - yt).max():.2e}")
    assert worst <= 1.0
    assert np.abs(yl - yt).max() <= 1e-3 * np.abs(yt).max()


def test_external_block_mode_equals_identity_map():
    M, B, D, L = 3, 2, 4, 128
    say(f"case external block mode M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 11, decay=32.0) * 0.3
    x = np.random.default_rng(12).standard_normal((L, B, D)).astype(np.float32)
    with fi.Context(_cuda(h), B, map=fi.MAP_IDENTITY, tau_mode=fi.TAU_FFT, chunk_direct=False) as ref:
        yref = ref.prefill(_cuda(x))
    with fi.Context(_cuda(h), B, map=fi.MAP_EXTERNAL, tau_mode=fi.TAU_FFT) as ext:
        ys = []
        for n in range(L):
            q = _cuda(x[n])
            for l in range(M):
                q = ext.layer_red(l, q).clone()   # identity block between layers
            ys.append(q)
            ext.tiles()
        yext = torch.stack(ys)
    assert torch.equal(yext, yref)


def test_chunks_and_single_positions_interleave():
    """Prefill and generation switch between whole chunks (one launch for the
    G positions between FFT positions) and single positions at every kind of
    boundary; every recorded output replays against the oracle, and the run
    agrees with one launch per position to rounding."""
    M, B, D, L = 3, 2, 5, 1024
    say(f"case chunk / position interleave M={M} B={B} D={D} L={L} G=32")
    h = _filters(M, D, L, 17, decay=128.0) * 0.3
    x = np.random.default_rng(18).standard_normal((45, B, D)).astype(np.float32)
    outs = []
    for chunk in (True, False):
        with fi.Context(_cuda(h), B, tau_split=5, record=True, chunk_direct=chunk) as ctx:
            ys = [ctx.prefill(_cuda(x))]                 # chunk 1..32, then 33..45 one by one
            ys.append(ctx.generate(100))                 # 46..64, chunks 65..128, 129..145
            ys.append(torch.stack([ctx.step() for _ in range(10)]))
            ys.append(ctx.generate(L - 155))             # ... up to L, the last chunk ends at L
            assert ctx.position == L
            outs.append(torch.cat(ys).cpu().numpy())
            worst = check_replay(h, ctx)
            say(f"  chunk={chunk} replay worst error/tolerance {worst:.3e}")
            assert worst <= 1.0
    rel = np.abs(outs[0] - outs[1]).max() / np.abs(outs[1]).max()
    say(f"  chunked vs per-position rel diff {rel:.2e}")
    assert rel <= 1e-3


@pytest.mark.parametrize("D", [515, 1103])
def test_chunk_workgroups_with_ragged_chain_counts(D):
    """More chains than CUs: several chains per chunk workgroup, the last
    workgroup short; 256-position chunks (taps h[2..255] in the helpers)."""
    M, B, L = 2, 1, 1024
    say(f"case chunk ragged M={M} B={B} D={D} L={L} G=256")
    h = _filters(M, D, L, 19, decay=200.0) * 0.1
    x = np.random.default_rng(20).standard_normal((L, B, D)).astype(np.float32)
    with fi.Context(_cuda(h), B, tau_split=8, record=True) as ctx:
        ctx.prefill(_cuda(x))
        chans = sorted(set([0, 1, 2, 3, D // 2, D - 4, D - 3, D - 2, D - 1]))
        worst = check_replay(h, ctx, chans=chans)
    say(f"  replay worst error/tolerance {worst:.3e}")
    assert worst <= 1.0


@pytest.mark.parametrize("M", [20, 23])
def test_deep_stacks_in_chunks(M):
    """The deepest stack kept in registers (M = 20) and one past it (M = 23: the chain reads its layers
    from LDS), three chains per chunk workgroup: 60 and 69 rows, so the last helper wave holds a part
    of a row group.  Teacher-forced prefill (positions in chunks) and a free-running generation with
    both maps tanh, each replayed layer by layer against the oracle."""
    B, D, L = 1, 700, 1024
    say(f"case deep stack in chunks M={M} B={B} D={D} L={L} G=256")
    h = _filters(M, D, L, 51, decay=150.0) * 0.1
    x = np.random.default_rng(52).standard_normal((L, B, D)).astype(np.float32)
    chans = [0, 1, 2, 3, 4, 5, 350, 696, 697, 698, 699]
    with fi.Context(_cuda(h), B, tau_split=8, record=True, map=fi.MAP_IDENTITY) as ctx:
        ctx.prefill(_cuda(x))
        worst = check_replay(h, ctx, chans=chans)
    say(f"  teacher-forced replay worst error/tolerance {worst:.3e}")
    assert worst <= 1.0
    with fi.Context(_cuda(h), B, tau_split=8, record=True) as ctx:
        ctx.set_input(_cuda(x[0]))
        y = ctx.generate(L).cpu().numpy()
        worst = check_replay(h, ctx, chans=chans)
    say(f"  free-running replay worst error/tolerance {worst:.3e}, max |y| {np.abs(y).max():.3g}")
    assert worst <= 1.0
    assert np.isfinite(y).all()


@pytest.mark.parametrize("L", [1, 2, 4, 8, 32])
def test_edge_lengths_and_ragged_chain_counts(L):
    M, B, D = 2, 3, 7
    say(f"case edge L={L} M={M} B={B} D={D}")
    h = _filters(M, D, L, 13)
    x = np.random.default_rng(14).standard_normal((L, B, D)).astype(np.float32)
    for tau in (fi.TAU_DIRECT, fi.TAU_FFT):
        with fi.Context(_cuda(h), B, tau_mode=tau, record=True, map=fi.MAP_IDENTITY) as ctx:
            ctx.prefill(_cuda(x))
            assert check_replay(h, ctx) <= 1.0
            with pytest.raises(fi.FiError):
                ctx.step(_cuda(x[0]))


@pytest.mark.parametrize("scale", [0.002, 0.05, 1.0])
def test_chunk_kernel_with_and_without_records_agree(scale):
    """The chunk kernel the bench runs (no records) against the one the oracle replay checks (records
    on): the same arithmetic, so the outputs agree bit for bit; and the recorded run replays against
    the oracle, with every layer's input (and the fed-back input) the tanh of the output before it
    to 2 ulp.  The scale picks the
    chains' tanh passes: 0.002 keeps every |y| below 0.125 (the first piece alone holds), 0.05 leaves
    that range but stays below 0.72 (the polynomial pass), 1.0 leaves that too (the full-tanh runs).
    The split is pinned: a calibrated one is timed per context and can differ between the two, and
    with it the chunk length and the order of the additions."""
    M, B, D, L = 3, 2, 37, 2048
    say(f"case chunk kernel records on/off scale={scale} M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 31, decay=200.0) * scale
    x1 = np.random.default_rng(32).standard_normal((B, D)).astype(np.float32)
    outs = []
    for rec in (False, True):
        with fi.Context(_cuda(h), B, record=rec, tau_split=8) as ctx:
            ctx.set_input(_cuda(x1))
            outs.append(ctx.generate(L).cpu().numpy())
            if rec:
                worst = check_replay(h, ctx)
                ulps = 0.0
                big = 0.0
                for l in range(M):
                    yl = ctx.history(l, 1).cpu().numpy().astype(np.float64)
                    big = max(big, float(np.abs(yl).max()))
                    # the next layer's inputs, or for the last layer the fed-back input of the next position
                    t = np.tanh(yl) if l + 1 < M else np.tanh(yl[:-1])
                    xn = ctx.history(l + 1, 0).cpu().numpy() if l + 1 < M else ctx.history(0, 0).cpu().numpy()[1:]
                    ulps = max(ulps, float((np.abs(xn - t) / np.maximum(np.abs(t) * 2.0 ** -23, 1e-45)).max()))
    say(f"  max |y| over all layers {big:.3g}; replay worst error/tolerance {worst:.3e}; "
        f"layer inputs vs tanh of the layer before: {ulps:.2f} x 2^-23 relative")
    assert worst <= 1.0
    assert ulps <= 2.0
    lo, hi = {0.002: (0.0, 0.125), 0.05: (0.125, 0.72), 1.0: (0.72, np.inf)}[scale]
    assert lo <= big < hi
    assert np.array_equal(outs[0], outs[1])


def test_schedule_and_stamps():
    M, B, D, L = 1, 1, 4, 64
    say(f"case schedule/stamps L={L}")
    h = _filters(M, D, L, 15)
    with fi.Context(_cuda(h), B) as ctx:
        for n in range(1, L + 1):
            q, _ = ctx.schedule(n)
            assert q == (-1 if n == L else (n & -n).bit_length() - 1)
        ctx.generate(L, want_y=False)
        st = ctx.stamps(1, L)
        assert (st > 0).all() and (np.diff(st) >= 0).all()
        ctx.reset()
        assert ctx.position == 0
        ctx.generate(3, want_y=False)
        assert ctx.position == 3


def test_stamps_with_chunks():
    """Positions run in chunks of 64 (first FFT class 6): every position is stamped in order,
    including a chunk's last position, which is stamped by its FFT gray block's last workgroup,
    also when a run stops right there."""
    M, B, D, L = 2, 1, 16, 1024
    say(f"case stamps with chunks M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 21, decay=64.0)
    with fi.Context(_cuda(h), B, tau_split=6) as ctx:
        assert ctx.schedule(64) == (6, fi.PATH_FFT)
        ctx.generate(64, want_y=False)
        st = ctx.stamps(1, 64)
        assert (st > 0).all() and (np.diff(st) >= 0).all()
        ctx.generate(L - 64, want_y=False)
        st = ctx.stamps(1, L)
        assert (st > 0).all() and (np.diff(st) >= 0).all()
        assert ctx.position == L


def test_binding_rejects_mismatched_tensors():
    """Shapes, dtypes and layouts that do not match the context are FI_EINVAL
    before any kernel runs; the context stays usable."""
    M, B, D, L = 1, 2, 5, 64
    say(f"case binding argument checks M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 41)
    with fi.Context(_cuda(h), B) as ctx:
        bad = [torch.zeros((B, D + 1), device="cuda"), torch.zeros((B, D), dtype=torch.float64, device="cuda"),
               torch.zeros((D, B), device="cuda").t(), torch.zeros((B * D,), device="cuda")]
        for t in bad:
            with pytest.raises(fi.FiError) as e:
                ctx.step(t)
            assert e.value.status == fi.FI_EINVAL
            with pytest.raises(fi.FiError):
                ctx.step(None, y=t)
        with pytest.raises(fi.FiError):
            ctx.prefill(torch.zeros((4, B + 1, D), device="cuda"))
        with pytest.raises(fi.FiError):
            ctx.generate(4, y=torch.zeros((3, B, D), device="cuda"))
        assert ctx.position == 0
        ctx.set_input(torch.zeros((B, D), device="cuda"))
        ctx.generate(4, want_y=False)
        assert ctx.position == 4
    with fi.DDContext(B, D, L) as dd:
        with pytest.raises(fi.FiError):
            dd.step(torch.zeros((B, D), device="cuda"), torch.zeros((B, D + 1), device="cuda"))
        with pytest.raises(fi.FiError):
            dd.run(torch.zeros((4, B, D), device="cuda"), torch.zeros((3, B, D), device="cuda"))
        assert dd.position == 0


def test_auto_split_is_timed_on_the_chunk_path():
    """With chunked positions, the calibrated split is the shortest chunk whose
    timed chunk (and FFT block) gives a modeled run within 1.5% of the cheapest;
    the per-position path keeps its per-class timing."""
    M, B, D, L = 2, 1, 64, 4096
    say(f"case chunk-path calibration M={M} B={B} D={D} L={L}")
    h = _filters(M, D, L, 43, decay=512.0) * 0.1
    with fi.Context(_cuda(h), B) as ctx:
        table = ctx.chunk_table()
        paths = [p for (_, p, _, _) in ctx.tau_table()]
    timed = [(g, uc, ur) for (g, uc, ur) in table if ur >= 0]
    assert [g for g, _, _ in timed] == list(range(2, 9))
    assert all(uc > 0 for _, uc, _ in timed)
    least = min(ur for _, _, ur in timed)
    best = min(g for g, _, ur in timed if ur <= least * 1.015)
    split = next(q for q, p in enumerate(paths) if p == fi.PATH_FFT)
    say(f"  modeled run per candidate {[(g, round(ur)) for g, _, ur in timed]}; split {split}")
    assert split == best
    with fi.Context(_cuda(h), B, chunk_direct=False) as ctx:
        assert all(ur < 0 for (_, _, ur) in ctx.chunk_table())
        assert any(ud > 0 for (_, _, ud, _) in ctx.tau_table())
