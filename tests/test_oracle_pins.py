"""Pins that tie the CPU oracle to the pages and to mathematics, not to itself.

Each check would fail for a plausible slip in the oracle: a dropped term, an
off-by-one index, a reversed filter, a wrong feedback shift, a missing map.
CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import block, relaxed, schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(L, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal(L) * scale).astype(np.float32)


def _scale(h, x):
    return float(np.abs(h.astype(np.float64)).sum() * np.abs(x.astype(np.float64)).max())


# --------------------------------------------------------------------------
# causal convolution: brute force, library routine, full-length FFT, closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 2, 3, 17, 64])
def test_conv_equals_toeplitz_and_numpy_convolve(L):
    h, x = _rand(L, 1), _rand(L, 2)
    y = oracle.conv_rows(h, x)
    T = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            T[t, s] = h[t - s]
    ref_toeplitz = T @ x.astype(np.float64)
    ref_np = np.convolve(h.astype(np.float64), x.astype(np.float64))[:L]
    tol = 1e-14 * max(_scale(h, x), 1e-30)
    assert np.max(np.abs(y - ref_toeplitz)) <= tol
    assert np.max(np.abs(y - ref_np)) <= tol


def test_conv_equals_full_length_fft():
    L = 4096
    h, x = _rand(L, 3) * np.exp(-np.arange(L) / 500.0).astype(np.float32), _rand(L, 4)
    y = oracle.conv_rows(h, x)
    H = np.fft.rfft(h.astype(np.float64), 2 * L)
    X = np.fft.rfft(x.astype(np.float64), 2 * L)
    ref = np.fft.irfft(H * X, 2 * L)[:L]
    assert np.max(np.abs(y - ref)) <= 1e-10 * _scale(h, x)


def test_conv_rows_batched_rows_are_independent():
    L, R = 300, 5
    h = np.stack([_rand(L, 10 + r) for r in range(R)])
    x = np.stack([_rand(L, 20 + r) for r in range(R)])
    y = oracle.conv_rows(h, x)
    for r in range(R):
        ref = np.convolve(h[r].astype(np.float64), x[r].astype(np.float64))[:L]
        assert np.max(np.abs(y[r] - ref)) <= 1e-12 * _scale(h[r], x[r])


def test_conv_closed_forms():
    L = 48
    x = _rand(L, 5)
    # h = delta_0: y = x exactly
    d0 = np.zeros(L, np.float32); d0[0] = 1
    assert np.array_equal(oracle.conv_rows(d0, x), x.astype(np.float64))
    # h = delta_k: y_t = x_{t-k}, zero before k
    for k in (1, 5, 47):
        dk = np.zeros(L, np.float32); dk[k] = 1
        ref = np.zeros(L); ref[k:] = x[:L - k]
        assert np.array_equal(oracle.conv_rows(dk, x), ref)
    # h = 1: prefix sums
    ones = np.ones(L, np.float32)
    assert np.allclose(oracle.conv_rows(ones, x), np.cumsum(x.astype(np.float64)), rtol=0, atol=1e-12)
    # h_k = 2^-k, x = 1: y_n (1-based n terms) = 2 - 2^(1-n), exact in fp64 for n <= 48
    geo = (0.5 ** np.arange(L)).astype(np.float32)
    n = np.arange(1, L + 1, dtype=np.float64)
    assert np.array_equal(oracle.conv_rows(geo, ones), 2.0 - 2.0 ** (1.0 - n))
    # h_k = r^k, x = 1 -> (1 - r^n)/(1 - r) up to the fp32 rounding of the taps
    r = 0.9
    L2 = 400
    geo9 = (r ** np.arange(L2)).astype(np.float32)
    n2 = np.arange(1, L2 + 1, dtype=np.float64)
    ref = (1 - r ** n2) / (1 - r)
    assert np.max(np.abs(oracle.conv_rows(geo9, np.ones(L2, np.float32)) - ref) / ref) < 1e-6


def test_conv_points_equal_library_convolution():
    L = 5000
    h, x = _rand(L, 6), _rand(L, 7)
    ts = np.array([0, 1, 2, 777, 2048, 4095, 4999])
    ref = np.convolve(h.astype(np.float64), x.astype(np.float64))[:L][ts]
    assert np.max(np.abs(oracle.conv_points(h, x, ts) - ref)) <= 1e-11 * _scale(h, x)


# --------------------------------------------------------------------------
# autoregressive stack: teacher forcing vs layerwise FFT, feedback fixed point,
# closed-form recurrences
# --------------------------------------------------------------------------

def _fft_conv(h, x):
    L = x.shape[-1]
    H = np.fft.rfft(np.asarray(h, np.float64), 2 * L)
    X = np.fft.rfft(np.asarray(x, np.float64), 2 * L)
    return np.fft.irfft(H * X, 2 * L)[..., :L]


def _filters(M, D, L, seed, decay=50.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((M, D, L)) * np.exp(-np.arange(L) / decay)).astype(np.float32)


def test_stack_teacher_forced_equals_layerwise_fft():
    M, D, L = 3, 4, 256
    f = _filters(M, D, L, 11)
    chans = np.array([0, 2, 3, 1])
    xg = np.random.default_rng(12).standard_normal((4, L)).astype(np.float32)
    y, x = oracle.stack(f, chans, xg[:, 0], L, x_given=xg)
    for k, c in enumerate(chans):
        xin = xg[k].astype(np.float64)
        for l in range(M):
            assert np.max(np.abs(x[k, l] - xin)) <= 1e-12
            ref = _fft_conv(f[l, c], xin)
            assert np.max(np.abs(y[k, l] - ref)) <= 1e-10 * (np.abs(f[l, c]).sum() * np.abs(xin).max())
            xin = np.tanh(ref)


def test_stack_single_layer_teacher_forced_equals_convolve():
    L = 512
    f = _filters(1, 2, L, 13)
    xg = np.random.default_rng(14).standard_normal((1, L)).astype(np.float32)
    y, _ = oracle.stack(f, [1], xg[:, 0], L, x_given=xg)
    ref = np.convolve(f[0, 1].astype(np.float64), xg[0].astype(np.float64))[:L]
    assert np.max(np.abs(y[0, 0] - ref)) <= 1e-11 * _scale(f[0, 1], xg[0])


def test_stack_feedback_is_a_fixed_point_of_teacher_forcing():
    """The feedback run's own layer-0 sequence, pushed through the stack by
    full-sequence FFT convolution, must reproduce every layer's outputs, and the
    next input must be tanh of the previous last-layer output (one-step shift)."""
    M, D, L = 2, 3, 300
    f = _filters(M, D, L, 15, decay=20.0)
    chans = np.array([0, 1, 2])
    x1 = np.array([0.3, -1.2, 2.0], np.float32)
    y, x = oracle.stack(f, chans, x1, L)
    for k, c in enumerate(chans):
        assert x[k, 0, 0] == np.float64(x1[k])
        assert np.max(np.abs(x[k, 0, 1:] - np.tanh(y[k, M - 1, :-1]))) <= 1e-15
        xin = x[k, 0]
        for l in range(M):
            ref = _fft_conv(f[l, c], xin)
            assert np.max(np.abs(y[k, l] - ref)) <= 1e-10 * np.abs(f[l, c]).sum()
            xin = np.tanh(ref)


def test_stack_feedback_delta0_scalar_recurrence():
    """h^l = a_l * delta_0 for every layer: x_{n+1} = tanh(a_{M-1} tanh(... tanh(a_0 x_n)))."""
    M, L = 3, 64
    a = [1.7, -0.8, 2.5]
    f = np.zeros((M, 1, L), np.float32)
    for l in range(M):
        f[l, 0, 0] = a[l]
    x1 = np.float32(0.9)
    y, x = oracle.stack(f, [0], [x1], L)
    xn = float(x1)
    for n in range(L):
        v = xn
        for l in range(M):
            yl = float(np.float32(a[l])) * v
            assert abs(y[0, l, n] - yl) <= 1e-15
            v = math.tanh(yl)
        xn = v


def test_stack_feedback_delta1_closed_form():
    """M=1, h = delta_1: y_n = x_{n-1}; the input alternates tanh^k(x_1) and 0."""
    L = 41
    f = np.zeros((1, 1, L), np.float32)
    f[0, 0, 1] = 1
    x1 = 1.3
    _, x = oracle.stack(f, [0], [x1], L)
    v = float(np.float32(x1))
    for n in range(L):          # 0-based n: odd positions (1-based) carry the chain
        if n % 2 == 0:
            assert abs(x[0, 0, n] - v) <= 1e-15
            v = math.tanh(v)
        else:
            assert x[0, 0, n] == 0.0


def test_stack_identity_map_single_layer_feedback_is_linear_recurrence():
    """With identity feedback and h = delta_0 * a, x_n = a^(n-1) x_1."""
    L = 20
    f = np.zeros((1, 1, L), np.float32)
    f[0, 0, 0] = 0.5
    y, x = oracle.stack(f, [0], [3.0], L, map_tanh=False, fb_tanh=False)
    assert np.allclose(x[0, 0], 3.0 * 0.5 ** np.arange(L), rtol=1e-15, atol=0)


def test_stack_f32_tracks_fp64_on_short_horizon():
    M, D, L = 2, 2, 64
    f = _filters(M, D, L, 16, decay=10.0)
    y64, _ = oracle.stack(f, [0, 1], [0.5, -0.5], L)
    y32, _ = oracle.stack_f32(f, [0, 1], [0.5, -0.5], L)
    assert np.max(np.abs(y64 - y32)) < 1e-4 * max(1.0, np.abs(y64).max())


# --------------------------------------------------------------------------
# schedule: coverage, counts and the pages' fractions
# --------------------------------------------------------------------------

def test_largest_pow2_dividing_small_values():
    assert [schedule.largest_pow2_dividing(i) for i in range(1, 17)] == \
        [1, 2, 1, 4, 1, 2, 1, 8, 1, 2, 1, 4, 1, 2, 1, 16]


@pytest.mark.parametrize("P", list(range(0, 11)))
def test_schedule_covers_every_pair_exactly_once(P):
    L = 2 ** P
    cover = np.zeros((L + 1, L + 1), np.int32)       # cover[t, s], 1-based
    for i, U, (lo, hi), (olo, ohi) in schedule.gray_tiles(L):
        assert 1 <= lo <= hi == i < olo == i + 1 <= ohi <= L
        cover[olo:ohi + 1, lo:hi + 1] += 1
    for i in schedule.red_cells(L):
        cover[i, i] += 1
    want = np.tril(np.ones((L, L), np.int32))         # every s <= t exactly once
    assert np.array_equal(cover[1:, 1:], want)


@pytest.mark.parametrize("logL", [4, 8, 11])
def test_prompt_inputs_dead_after_prefill_only_for_top_runs(logL):
    """After a prefill of P positions has run every gray block after n <= P, a later
    block (n > P) still reads an input at or before P unless P = L - L/2^k: the prompt's
    activations can be dropped on this schedule exactly for P = L/2, 3L/4, ... (the
    relative schedule the rebuttal describes would allow it for every P)."""
    L = 2 ** logL
    tiles = list(schedule.gray_tiles(L))
    top_runs = {L - L // 2 ** k for k in range(1, logL + 1)}
    for P in range(1, L):
        reaches_back = any(i > P and lo <= P for i, U, (lo, hi), _ in tiles)
        assert reaches_back == (P not in top_runs), P


@pytest.mark.parametrize("P", [1, 4, 10, 16])
def test_schedule_counts_match_proposition_1(P):
    facts = json.load(open(os.path.join(GOLDEN, "schedule_facts.json")))
    assert facts["calls_per_class"] == "2^(P-1-q)"
    L = 2 ** P
    count = {}
    area = 0
    for i in range(1, L):
        U = schedule.largest_pow2_dividing(i)
        count[U] = count.get(U, 0) + 1
        area += U * U
    assert sum(count.values()) == L - 1
    for q in range(P):
        assert count.get(2 ** q, 0) == 2 ** (P - 1 - q)
    assert area == L * (L - 1) // 2


@pytest.mark.parametrize("L", [1, 2, 16, 100, 512])
def test_data_dependent_tiling_covers_every_pair_once_in_time(L):
    """Two-sided tiling for filters that arrive with the data: every pair (i, j) with i + j < L
    exactly once, each formed at a step n with both inputs known (max(i, j) <= n) and, for a
    block, its target still ahead (i + j > n); red cells at their own target."""
    cover = np.zeros((L, L), np.int32)
    for n in range(L):
        for i, j in schedule.dd_red_pairs(n):
            assert max(i, j) == n == i + j
            cover[i, j] += 1
        for kind, p, xl, hl in schedule.dd_blocks(n):
            assert xl + p - 1 <= n and hl + p - 1 <= n and xl + hl > n
            assert xl + hl + 2 * p - 2 >= xl + hl
            hi_i, hi_j = min(xl + p, L), min(hl + p, L)
            cover[xl:hi_i, hl:hi_j] += 1
    want = np.fliplr(np.triu(np.ones((L, L), np.int32)))      # i + j <= L - 1
    want_mask = np.add.outer(np.arange(L), np.arange(L)) < L
    assert np.array_equal(cover[want_mask], np.ones(int(want_mask.sum()), np.int32))
    assert want.sum() == want_mask.sum()


def test_data_dependent_tiling_runs_two_products_per_band_block():
    """The pages' account of the modification: a step forms two same-size products where the
    fixed-filter tiling forms one (the squares at 2p - 1 excepted); the products' total area is
    the number of pairs, L(L+1)/2 minus the red cells, over all steps up to L = 2^10 - 1."""
    L = 1024
    area = 0
    for n in range(L):
        blocks = list(schedule.dd_blocks(n))
        sizes = {}
        for kind, p, xl, hl in blocks:
            sizes.setdefault(p, []).append(kind)
            area += p * p
        for p, kinds in sizes.items():
            assert sorted(kinds) in (["square"], ["h", "x"])
            assert (kinds == ["square"]) == (n + 1 == 2 * p)
    # pairs (i, j), i, j >= 1, with max(i, j) < L: blocks never stop short of L
    assert area == (L - 1) * (L - 1)


def test_schedule_fractions_match_pages():
    facts = json.load(open(os.path.join(GOLDEN, "schedule_facts.json")))
    P = 17
    L = 2 ** P
    Us = np.array([schedule.largest_pow2_dividing(i) for i in range(1, L)])
    frac_le4 = float(np.mean(Us <= 4))
    frac_le8 = float(np.mean(Us <= 8))
    assert abs(frac_le4 - facts["fraction_tiles_U_le_4"]) < 1e-4
    assert abs(frac_le8 - facts["fraction_tokens_U_le_8"]) < 1e-4


# --------------------------------------------------------------------------
# Algorithm 1 tile by tile reproduces the definition (direct and circular FFT)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 2, 8, 64, 256])
@pytest.mark.parametrize("tile", ["direct", "fft"])
def test_relaxed_algorithm_equals_definition(L, tile):
    if tile == "direct" and L > 64:
        pytest.skip("pure-Python direct tiles are slow; fft covers the larger size")
    h, x = _rand(L, 30), _rand(L, 31)
    z = relaxed.relaxed_conv(h, x, tile=tile)
    ref = oracle.conv_rows(h, x)
    assert np.max(np.abs(z - ref)) <= 1e-12 * _scale(h, x)


@pytest.mark.parametrize("U", [1, 2, 4, 16, 128, 1024])
def test_circular_2U_trick_keeps_upper_half_exact(U):
    r = np.random.default_rng(U)
    a = r.standard_normal(U)
    g = r.standard_normal(2 * U)
    pad = np.concatenate([a, np.zeros(U)])
    circ = np.fft.ifft(np.fft.fft(pad) * np.fft.fft(g)).real[U:]
    lin = np.array([sum(a[j] * g[m - j] for j in range(U)) for m in range(U, 2 * U)])
    assert np.max(np.abs(circ - lin)) <= 1e-12 * np.abs(a).max() * np.abs(g).sum()
    # and the lower half is NOT the linear result in general (wrap-around)
    if U >= 2:
        lin_low = np.array([sum(a[j] * g[m - j] for j in range(min(U, m + 1))) for m in range(U)])
        circ_low = np.fft.ifft(np.fft.fft(pad) * np.fft.fft(g)).real[:U]
        assert np.max(np.abs(circ_low - lin_low)) > 1e-6


# --------------------------------------------------------------------------
# Hyena-style block
# --------------------------------------------------------------------------

def test_gelu_matches_textbook_normal_cdf():
    t = json.load(open(os.path.join(GOLDEN, "normal_cdf.json")))
    z = np.array(t["z"])
    phi = np.array(t["Phi"])
    assert np.max(np.abs(block.gelu(z) - z * phi)) < 1e-15 * 4


def test_rmsnorm_properties():
    r = np.random.default_rng(40)
    z = r.standard_normal((3, 768))
    a = block.rmsnorm(z)
    ms = np.mean(z * z, axis=-1)
    assert np.allclose(np.mean(a * a, axis=-1), ms / (ms + block.RMS_EPS), rtol=1e-14)
    assert np.allclose(block.rmsnorm(7.5 * z), a, rtol=1e-6)        # scale invariance (eps aside)
    assert np.allclose(np.sign(a), np.sign(z))


def test_block_generate_structured_weights_closed_form():
    """W = [I|I|I] (u=v=w=x), W1 = [I 0 0 0], W2 = [I;0;0;0]: per position
    q = x^2, c = causal conv(h, q), a = RMSNorm(GELU(x*c)), next x = tanh(a)."""
    M, B, D, L = 1, 2, 3, 24
    r = np.random.default_rng(41)
    f = (r.standard_normal((M, D, L)) * 0.3).astype(np.float32)
    I = np.eye(D)
    W = np.concatenate([I, I, I], axis=1)[None]
    W1 = np.concatenate([I, np.zeros((D, 3 * D))], axis=1)[None]
    W2 = np.concatenate([I, np.zeros((3 * D, D))], axis=0)[None]
    x1 = r.standard_normal((B, D))
    out = block.generate(f, W, W1, W2, x1, L)
    x = np.zeros((L, B, D))
    x[0] = x1
    x[1:] = np.tanh(out["a"][:-1, 0])
    q = x * x
    assert np.allclose(out["q"][:, 0], q, rtol=0, atol=1e-13)
    for b in range(B):
        for d in range(D):
            c = np.convolve(f[0, d].astype(np.float64), q[:, b, d])[:L]
            assert np.allclose(out["c"][:, 0, b, d], c, rtol=0, atol=1e-12)
    g = block.gelu(x * out["c"][:, 0])
    ref_a = g / np.sqrt(np.mean(g * g, axis=-1, keepdims=True) + 1e-6)
    assert np.allclose(out["a"][:, 0], ref_a, rtol=0, atol=1e-12)


def test_block_split_order_u_v_w():
    """Column blocks of x W are u, v, w in that order: only v's block reaches the gate."""
    D = 4
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    W = np.zeros((D, 3 * D))
    W[:, D:2 * D] = np.eye(D)        # v = x, u = w = 0
    q, v = block.project(x, W)
    assert np.array_equal(q, np.zeros((1, D))) and np.array_equal(v, x)
    W = np.zeros((D, 3 * D))
    W[:, 0:D] = np.eye(D)
    W[:, 2 * D:] = 2 * np.eye(D)     # u = x, w = 2x, v = 0
    q, v = block.project(x, W)
    assert np.array_equal(q, 2 * x * x) and np.array_equal(v, np.zeros((1, D)))
