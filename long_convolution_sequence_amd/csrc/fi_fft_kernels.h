// FFT gray-block kernels and the filter spectra they read: the transform
// of every block-size class in one workgroup (k_fft_tile), the class two
// halves wide (k_fft_tile2), and the split classes (k_fft_sub_fwd/inv).
//
// Flash Inference (arXiv 2410.12982), summary page, "Zirkulaere
// Faltungs-Trick" and "FFT-Vorberechnung": each gray block is a 2U-point
// circular convolution against a cached filter spectrum, of which the upper
// half is exact.
#pragma once
#include "fi_device.h"
#include "fi_fft.h"

namespace fi {

// ---------------------------------------------------------------------------
// Gray blocks of all layers by FFT, U = 2^LOGN (complex transform of U points
// carries the 2U-point real circular convolution).  One team of TT threads per
// (l, b, c) block; the red cells at n have already run.
//   spec: per (l, c), U/2 float4 in pair order (see k_spectrum), scaled by 1/U.
// ---------------------------------------------------------------------------
// One gray block of edge N = 2^LOGN for the calling team (TT threads, lt
// its thread): the block's N inputs at xsrc (N/2 float2), times the filter
// spectrum sp (N/2 float4 in pair order), transformed back.  On return this
// thread holds in v[HALF0 + m] the outputs at float2 index lt + (m << QLOG0)
// of the exact upper half (targets n+1 .. n+N of the block after n).  Every
// thread of the workgroup calls it (it synchronises); inactive teams compute
// on zeros.  X: the team's LDS.  before_last() runs just before the last
// inverse stage group (a caller issues its loads of the targets there, so
// that the group's arithmetic covers their latency).
template <int LOGN, bool SPEC2 = (LOGN == 13), typename BeforeLast>
__device__ __forceinline__ void fft_block(const Dev &p, float2 *X, int lt, bool active, const float2 *xsrc,
                                          const float4 *sp, float2 (&v)[1 << FftShape<LOGN>::R0],
                                          BeforeLast &&before_last) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
#pragma unroll
    for (int m = 0; m < HALF0; ++m) {
        v[m] = active ? xsrc[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
        v[m + HALF0] = make_float2(0.f, 0.f);
    }
    dif_group<R0, true>(v, lt, LOGN, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt) + lpad_off(m, QLOG0)] = v[m];
    // this thread's spectrum pairs, loaded late: held across the whole forward
    // transform they would cost the registers of a fourth wave per SIMD.  When
    // the last stage group is short (fewer than four stages), they are issued
    // before it, so that it covers part of their latency; with SPEC2 (the
    // gray blocks of 2^13 points, whose last group has one stage) one group
    // earlier still, which their registers allow (569 -> 547 us for that
    // class; slower for 2^14, and a caller that runs two blocks spills).
    constexpr int NP = S::NPASS;
    constexpr bool EARLY = NP >= 2 && LOGN - 4 * (NP - 1) < 4;
    constexpr int SPL = SPEC2 && NP >= 3 ? NP - 2 : NP - 1;   // group before which they are issued
    forward_groups<LOGN, 1, EARLY ? SPL : NP>(X, lt, p.twid, p.logNT);
    constexpr int PAIRS = (N / 2 + TT - 1) / TT;
    float4 gs[PAIRS];
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        gs[m] = (active && e < N / 2) ? sp[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (EARLY) forward_groups<LOGN, SPL, NP>(X, lt, p.twid, p.logNT);
    __syncthreads();

    // bins of the real transform times the filter spectrum, re-packed for the
    // inverse; the items' pair twiddles are all read first, so that their
    // latency is paid once (item 0 reads an unused entry)
    static_assert((N / 2) % TT == 0, "items per thread");
    float2 wp[PAIRS];
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) wp[m] = p.ptw[N / 2 + lt + m * TT];
    const PairLds pl = pair_lds<LOGN>(lt);
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        const float4 g = gs[m];
        if (e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            const float Z0 = (C0.x + C0.y) * g.x;
            const float ZN = (C0.x - C0.y) * g.y;
            X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
            X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w));
        } else {
            const SlotPair sl = item_lds<LOGN, TT>(pl, lt, m);
            const int p1 = sl.a, p2 = sl.b;
            const float2 W = wp[m];
            float2 A1, A2, D1, D2;
            real_bins(X[p1], X[p2], W, A1, A2);
            pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2);
            X[p1] = D1;
            X[p2] = D2;
        }
    }
    const float2 wi = group_root<LOGN, S::NPASS - 1>(lt, p.twid, p.logNT);
    __syncthreads();
    const float2 w0 = inverse_groups<LOGN, S::NPASS - 1>(X, lt, p.twid, p.logNT, wi);
    before_last();
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt) + lpad_off(m, QLOG0)];
    dit_group_w<R0>(v, w0);
}

// Four waves per SIMD is what the LDS allows at every size from 2^8 on; the
// register budget is held to that.
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) __attribute__((amdgpu_waves_per_eu(LOGN >= 8 ? 4 : 1)))
k_fft_tile(Dev p, int rd, const float4 *__restrict__ spec, int advance) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long n = position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L || n % N != 0 || n + N > p.L) return;  // uniform guard, as in k_direct
    const long long ntiles = (long long)p.M * p.B * p.D;
    const long long tile = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = tile < ntiles;
    float2 *X = smem + team * lds_len(N);
    const int c = (int)(tile % p.D);
    const int l = (int)(tile / ((long long)p.D * p.B));
    const size_t row = (size_t)tile * (size_t)p.L;
    const float2 *xsrc = reinterpret_cast<const float2 *>(p.buf + row + t - N + 1);
    float2 *adst = reinterpret_cast<float2 *>(p.buf + row + t + 1);
    const float4 *sp = spec + ((size_t)l * p.D + c) * (N / 2);
    float2 v[1 << R0];
    // the pending sums, like the spectrum, are read late: during the last
    // inverse stage group
    float2 acc[HALF0];
    fft_block<LOGN>(p, X, lt, active, xsrc, sp, v, [&]() {
#pragma unroll
        for (int m = 0; m < HALF0; ++m) acc[m] = active ? adst[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
    });
    if (active) {
#pragma unroll
        for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    }
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// Eager prefill, far part (the pages' prefill: the prompt's inputs of a layer
// are all known at once).  Every gray block of edge N = 2^LOGN after a
// position n <= P, n = (2j+1) N with j = blockIdx.y, for the B*D rows of layer
// l: the same transform as k_fft_tile; targets t <= P add into the prefill
// sums pre[(b, c)][t-1] (row stride pstride), later ones into the pending sums
// of the history.  P is even, so no float2 of outputs straddles it.
// ---------------------------------------------------------------------------
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) __attribute__((amdgpu_waves_per_eu(LOGN >= 8 ? 4 : 1)))
k_pre_fft(Dev p, const float4 *__restrict__ spec, int l, long long P, float *pre, int pstride) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long n = (2LL * blockIdx.y + 1) * N;
    const long long BD = (long long)p.B * p.D;
    const long long k = (long long)blockIdx.x * S::PER_BLOCK + team;   // (b, c) of layer l
    const bool active = k < BD && n <= P && n + N <= p.L;
    float2 *X = smem + team * lds_len(N);
    const long long kk = active ? k : 0;
    const int c = (int)(kk % p.D);
    const size_t row = ((size_t)l * BD + kk) * (size_t)p.L;
    const float2 *xsrc = reinterpret_cast<const float2 *>(p.buf + row + n - N);
    const float4 *sp = spec + ((size_t)l * p.D + c) * (N / 2);
    float2 v[1 << R0];
    fft_block<LOGN>(p, X, lt, active, xsrc, sp, v, []() {});
    if (active) {
#pragma unroll
        for (int m = 0; m < HALF0; ++m) {
            const long long s0 = n + 2LL * (lt + (m << QLOG0));   // slot of target s0 + 1
            float2 *dst = reinterpret_cast<float2 *>(s0 < P ? pre + (size_t)kk * pstride + s0 : p.buf + row + s0);
            *dst = cadd(*dst, v[m + HALF0]);
        }
    }
}

// ---------------------------------------------------------------------------
// Filter spectra ("FFT-Vorberechnung"): for every (l, c) row, the 2N-point real
// FFT of the taps g_r = h[goff + r], r in [0, 2N), stored in pair order
// (item e of pair_slot, bin j = pair_slot(e).j):
//   spec[0] = (G_0, G_N, Re G_{N/2}, Im G_{N/2}) / N
//   spec[e] = (G_j, G_{N-j}) / N,  0 < e < N/2.
// The 1/N folds the inverse transform's normalisation into the spectrum.
// ---------------------------------------------------------------------------
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) k_spectrum(Dev p, float4 *__restrict__ spec,
                                                                  long long goff, long long row_stride) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long rows = (long long)p.M * p.D;
    const long long rowi = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = rowi < rows;
    float2 *X = smem + team * lds_len(N);
    const float2 *src = reinterpret_cast<const float2 *>(p.filt + (size_t)rowi * (size_t)p.L + goff);
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = active ? src[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
    dif_group<R0>(v, lt, LOGN, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt) + lpad_off(m, QLOG0)] = v[m];
    forward_groups<LOGN, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    const float inv = 1.0f / (float)N;
    float4 *dst = spec + (size_t)rowi * (size_t)row_stride;
    for (int e = lt; e < N / 2 && active; e += TT) {
        if (e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            dst[0] = make_float4((C0.x + C0.y) * inv, (C0.x - C0.y) * inv, Ch.x * inv, -Ch.y * inv);
        } else {
            const PairSlot ps = pair_slot(LOGN, e);
            float2 A1, A2;
            real_bins(X[lpad(ps.pj)], X[lpad(ps.pm)], p.ptw[N / 2 + e], A1, A2);
            dst[e] = make_float4(A1.x * inv, A1.y * inv, A2.x * inv, A2.y * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// Transforms of 2M points (M = 2^LOGM) carried by their two M-point halves
// in turn (odd bins, then even bins; see odd_slot), so that only M points are
// ever in LDS.  In the item order of both halves a spectrum takes M float4:
// M/2 even-half items (pair_slot order, item 0 = (G_0, G_2M, G_M)), then M/2
// odd-half items.
// ---------------------------------------------------------------------------

// Forward transform of one half into X (bins bit-reversed, no trailing
// barrier).  Input: c = lo + hi (HI) or lo; the odd half takes c W_{2M}^m.
template <int LOGM, bool ODD, bool HI>
__device__ __forceinline__ void half_forward(const Dev &p, float2 *X, int lt, bool active, const float2 *lo,
                                             const float2 *hi) {
    using S = FftShape<LOGM>;
    constexpr int R0 = S::R0, QLOG0 = S::QLOG0;
    static_assert(R0 == 4, "two-half transforms have M >= 16");
    // W_{2M}^i at i = lt + m M/16 is W_{2M}^lt W_32^m
    const float2 wl = ODD ? twiddle(p.twid, p.logNT, LOGM + 1, lt) : make_float2(1.f, 0.f);
    float2 v[16];
    static_for<0, 16>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const int i = lt + (m << QLOG0);
        float2 c = active ? lo[i] : make_float2(0.f, 0.f);
        if constexpr (HI) {
            const float2 b = active ? hi[i] : make_float2(0.f, 0.f);
            c = ODD ? csub(c, b) : cadd(c, b);
        }
        v[m] = ODD ? mul_w32<m>(cmul(c, wl)) : c;
    });
    dif_group<R0>(v, lt, LOGM, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < 16; ++m) X[lpad(lt) + lpad_off(m, QLOG0)] = v[m];
    forward_groups<LOGM, 1, S::NPASS, false>(X, lt, p.twid, p.logNT);
}

// Inverse transform of one half from X (items already re-packed; the caller
// has synchronised) and its accumulation into dst[0..M): the odd half
// subtracts W_{2M}^{-m} v, the even half adds v.  The roots are read after
// the barriers here: held across them, they spill in these kernels.
template <int LOGM, bool ODD>
__device__ __forceinline__ void half_inverse_acc(const Dev &p, float2 *X, int lt, bool active, float2 *dst) {
    using S = FftShape<LOGM>;
    constexpr int R0 = S::R0, QLOG0 = S::QLOG0;
    const float2 w0 = inverse_groups<LOGM, S::NPASS - 1, false>(X, lt, p.twid, p.logNT, make_float2(1.f, 0.f));
    float2 v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = X[lpad(lt) + lpad_off(m, QLOG0)];
    dit_group_w<R0>(v, w0);
    if (!active) return;
    const float2 wl = ODD ? twiddle(p.twid, p.logNT, LOGM + 1, lt) : make_float2(1.f, 0.f);
    // in four runs of four, so that the accumulators never all occupy registers
    static_for<0, 4>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        float2 acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = dst[lt + ((4 * r + k) << QLOG0)];
        static_for<0, 4>([&](auto kc) {
            constexpr int m = 4 * r + decltype(kc)::value;
            const float2 a = acc[decltype(kc)::value];
            dst[lt + (m << QLOG0)] = ODD ? csub(a, mul_w32c<m>(cmulc(v[m], wl))) : cadd(a, v[m]);
        });
        asm volatile("" ::: "memory");
    });
}

template <int LOGM, bool ODD>
__device__ __forceinline__ PairSlot half_slot(int e) {
    return ODD ? odd_slot(LOGM, e) : pair_slot(LOGM, e);
}
template <int LOGM, bool ODD>
__device__ __forceinline__ float2 half_w(const Dev &p, int e) {
    return (ODD ? p.optw : p.ptw)[(1 << (LOGM - 1)) + e];
}

// Real bins of item e of a forward half in X, unscaled.
template <int LOGM, bool ODD>
__device__ __forceinline__ float4 half_bins(const Dev &p, const float2 *X, int e) {
    if (!ODD && e == 0) {
        const float2 C0 = X[0];
        const float2 Ch = X[lpad(1)];
        return make_float4(C0.x + C0.y, C0.x - C0.y, Ch.x, -Ch.y);
    }
    const PairSlot ps = half_slot<LOGM, ODD>(e);
    float2 A1, A2;
    real_bins(X[lpad(ps.pj)], X[lpad(ps.pm)], half_w<LOGM, ODD>(p, e), A1, A2);
    return make_float4(A1.x, A1.y, A2.x, A2.y);
}

// ---------------------------------------------------------------------------
// Gray blocks of U = 2M positions, M = 2^LOGM the widest one-workgroup
// transform: each half multiplies its bins by the matching half of the filter
// spectrum, transforms back and adds its part of the block's upper half into
// the accumulators, z = e - W_U^{-m} o for outputs m < M (the accumulators
// are read and written once per half, in that fixed order).
//   spec: per (l, c), M float4 in the two-half item order, scaled by 1/U.
// ---------------------------------------------------------------------------
template <int LOGM, bool ODD>
__device__ __forceinline__ void tile2_half(const Dev &p, float2 *X, int lt, bool active, const float2 *xsrc,
                                           float2 *adst, const float4 *sp) {
    using S = FftShape<LOGM>;
    constexpr int M = S::N, TT = S::TT;
    half_forward<LOGM, ODD, false>(p, X, lt, active, xsrc, nullptr);
    constexpr int PAIRS = (M / 2 + TT - 1) / TT;
    float4 gs[PAIRS];
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        gs[m] = (active && e < M / 2) ? sp[(ODD ? M / 2 : 0) + e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const PairLds pl = pair_lds<LOGM>(lt);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        if (e >= M / 2) break;
        const float4 g = gs[m];
        if (!ODD && e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            const float Z0 = (C0.x + C0.y) * g.x;
            const float ZN = (C0.x - C0.y) * g.y;
            X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
            X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w));
        } else {
            int p1, p2;
            if constexpr (ODD) {
                // odd half: positions 2e and M-1-2e (odd_slot), linear in m
                p1 = lpad(2 * lt) + lpad_off(m, FftShape<LOGM>::QLOG0 + 1);
                p2 = lpad(M - 1 - 2 * lt) - lpad_off(m, FftShape<LOGM>::QLOG0 + 1);
            } else {
                const SlotPair sl = item_lds<LOGM, TT>(pl, lt, m);
                p1 = sl.a;
                p2 = sl.b;
            }
            const float2 W = half_w<LOGM, ODD>(p, e);
            float2 A1, A2, D1, D2;
            real_bins(X[p1], X[p2], W, A1, A2);
            pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2);
            X[p1] = D1;
            X[p2] = D2;
        }
    }
    __syncthreads();
    half_inverse_acc<LOGM, ODD>(p, X, lt, active, adst);
}

template <int LOGM>
__global__ void __launch_bounds__(FftShape<LOGM>::TPB) __attribute__((amdgpu_waves_per_eu(4)))
k_fft_tile2(Dev p, int rd, const float4 *__restrict__ spec, int advance) {
    using S = FftShape<LOGM>;
    constexpr int M = S::N, TT = S::TT;
    constexpr long long U = 2LL * M;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long n = position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    const long long ntiles = (long long)p.M * p.B * p.D;
    const long long tile = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = tile < ntiles;
    float2 *X = smem + team * lds_len(M);
    const int c = (int)(tile % p.D);
    const int l = (int)(tile / ((long long)p.D * p.B));
    const size_t row = (size_t)tile * (size_t)p.L;
    const float2 *xsrc = reinterpret_cast<const float2 *>(p.buf + row + t - U + 1);
    float2 *adst = reinterpret_cast<float2 *>(p.buf + row + t + 1);
    const float4 *sp = spec + ((size_t)l * p.D + c) * M;
    tile2_half<LOGM, true>(p, X, lt, active, xsrc, adst, sp);
    __syncthreads();  // the even half reuses the LDS
    tile2_half<LOGM, false>(p, X, lt, active, xsrc, adst, sp);
    finish_position(p, n, advance);
}

// Eager prefill, far part for the two-half class (U = 2M): the gray blocks of
// edge U after positions n = (2j+1) U <= P (j = blockIdx.y) whose targets all
// lie inside the prompt (n + U <= P), for the B*D rows of layer l, added into
// the prefill sums pre[(b, c)][t-1].  Same transform as k_fft_tile2.
template <int LOGM>
__global__ void __launch_bounds__(FftShape<LOGM>::TPB) __attribute__((amdgpu_waves_per_eu(4)))
k_pre_fft2(Dev p, const float4 *__restrict__ spec, int l, long long P, float *pre, int pstride) {
    using S = FftShape<LOGM>;
    constexpr int M = S::N, TT = S::TT;
    constexpr long long U = 2LL * M;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long n = (2LL * blockIdx.y + 1) * U;
    if (n + U > P) return;                         // uniform guard: targets past the prompt are not ours
    const long long BD = (long long)p.B * p.D;
    const long long k = (long long)blockIdx.x * S::PER_BLOCK + team;   // (b, c) of layer l
    const bool active = k < BD;
    float2 *X = smem + team * lds_len(M);
    const long long kk = active ? k : 0;
    const int c = (int)(kk % p.D);
    const size_t row = ((size_t)l * BD + kk) * (size_t)p.L;
    const float2 *xsrc = reinterpret_cast<const float2 *>(p.buf + row + n - U);
    float2 *adst = reinterpret_cast<float2 *>(pre + (size_t)kk * pstride + n);
    const float4 *sp = spec + ((size_t)l * p.D + c) * M;
    tile2_half<LOGM, true>(p, X, lt, active, xsrc, adst, sp);
    __syncthreads();  // the even half reuses the LDS
    tile2_half<LOGM, false>(p, X, lt, active, xsrc, adst, sp);
}

// Filter spectra in the two-half item order: for every (l, c) row the taps
// g_r = h[goff + r], r in [0, 4M), packed into 2M complex points, scaled by
// 1/(2M), at spec + row * row_stride.
template <int LOGM>
__global__ void __launch_bounds__(FftShape<LOGM>::TPB) k_spectrum2(Dev p, float4 *__restrict__ spec, long long goff,
                                                                   long long row_stride) {
    using S = FftShape<LOGM>;
    constexpr int M = S::N, TT = S::TT;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long rows = (long long)p.M * p.D;
    const long long rowi = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = rowi < rows;
    float2 *X = smem + team * lds_len(M);
    const float2 *src = reinterpret_cast<const float2 *>(p.filt + (size_t)rowi * (size_t)p.L + goff);
    float4 *dst = spec + (size_t)rowi * (size_t)row_stride;
    const float inv = 1.0f / (float)(2 * M);
    static_for<0, 2>([&](auto hc) {
        constexpr bool ODD = decltype(hc)::value == 0;
        __syncthreads();  // the previous half's reads of X are done
        half_forward<LOGM, ODD, true>(p, X, lt, active, src, src + M);
        __syncthreads();
        for (int e = lt; e < M / 2 && active; e += TT) {
            const float4 b = half_bins<LOGM, ODD>(p, X, e);
            dst[(ODD ? M / 2 : 0) + e] = make_float4(b.x * inv, b.y * inv, b.z * inv, b.w * inv);
        }
    });
}

// ---------------------------------------------------------------------------
// Gray blocks wider than one workgroup's LDS transform (U = K * V, V = 2^LOGV).
// The block is split into K input sub-blocks i and K output sub-blocks o of
// V positions; sub-block i reaches sub-block o through taps offset by
// d*V, d = K + o - i (1 <= d <= 2K-1), and each such pair is again a
// length-2V circular convolution whose upper half is exact.  The sum over i is
// taken in frequency space, so each output sub-block needs one inverse
// transform.  Spectra: per (l, c), 2K-1 spectra (d = 1..2K-1) of the taps
// h[(d-1)V .. (d+1)V-1], each V/2 float4 in pair order.
//
// k_fft_sub_fwd: per (l, b, c, i), the real bins of the zero-padded input
// sub-block i, stored in pair order in `scratch` ([tile][i][V/2] float4).
// ---------------------------------------------------------------------------
// Workgroup w of a grid of T * K sub-block workgroups -> (tile, sub-block).
// Consecutive workgroup ids go to the eight XCDs in turn, so the K
// workgroups of one tile are given ids 8 apart: they run on one XCD at about
// the same time and share its L2 for the spectra they all read.
__device__ __forceinline__ void xcd_tile(long long w, long long T, int K, long long &tile, int &sub) {
    const long long full = (T / 8) * 8 * K;
    if (w < full) {
        const long long slot = w / 8;
        tile = (slot / K) * 8 + (w % 8);
        sub = (int)(slot % K);
    } else {
        tile = (full / K) + (w - full) / K;
        sub = (int)((w - full) % K);
    }
}

template <int LOGV>
__global__ void __launch_bounds__(FftShape<LOGV>::TPB) k_fft_sub_fwd(Dev p, int rd, float4 *__restrict__ scratch,
                                                                     int K) {
    using S = FftShape<LOGV>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    static_assert(S::PER_BLOCK == 1, "sub-block transforms fill a workgroup");
    __shared__ float2 smem[S::LDS];
    const int lt = threadIdx.x;
    const long long U = (long long)K * N;
    const long long n = position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    long long tile;
    int i;
    xcd_tile(blockIdx.x, (long long)p.M * p.B * p.D, K, tile, i);
    const size_t row = (size_t)tile * (size_t)p.L;
    const float2 *xsrc = reinterpret_cast<const float2 *>(p.buf + row + t - U + 1 + (long long)i * N);
    float2 *X = smem;
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) {
        v[m] = xsrc[lt + (m << QLOG0)];
        v[m + HALF0] = make_float2(0.f, 0.f);
    }
    dif_group<R0, true>(v, lt, LOGV, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt) + lpad_off(m, QLOG0)] = v[m];
    forward_groups<LOGV, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    float4 *dst = scratch + ((size_t)tile * K + i) * (N / 2);
    // the items' pair twiddles first (item 0 reads an unused entry)
    constexpr int PAIRS = N / 2 / TT;
    static_assert((N / 2) % TT == 0, "items per thread");
    float2 wp[PAIRS];
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) wp[m] = p.ptw[N / 2 + lt + m * TT];
    const PairLds pl = pair_lds<LOGV>(lt);
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        if (e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            dst[0] = make_float4(C0.x + C0.y, C0.x - C0.y, Ch.x, -Ch.y);
        } else {
            const SlotPair sl = item_lds<LOGV, TT>(pl, lt, m);
            float2 A1, A2;
            real_bins(X[sl.a], X[sl.b], wp[m], A1, A2);
            dst[e] = make_float4(A1.x, A1.y, A2.x, A2.y);
        }
    }
}

// Raw buffer load of 16 bytes at byte offset voff + soff of resource r
// (voff per lane, soff scalar); reads past the resource's size return zeros.
// Word 3 of a raw buffer resource on this architecture.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ float4 buffer_load4(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// An empty statement that the compiler must place after the values of Z are
// formed and that no memory access crosses.
template <int CH>
__device__ __forceinline__ void hold_after(float4 (&Z)[CH]) {
#pragma unroll
    for (int m = 0; m < CH; ++m) asm volatile("" : "+v"(Z[m].x), "+v"(Z[m].y), "+v"(Z[m].z), "+v"(Z[m].w)::"memory");
}

// k_fft_sub_inv: per (l, b, c, o), Z = sum_i A_i * G_{K+o-i}, then the inverse
// transform and accumulation of its exact upper half into output sub-block o.
// One launch covers output sub-blocks o0 .. o0+nO-1.  nfix > 0 names the
// position directly (a launch that runs after later positions have already
// overwritten the position slots).
// KT > 0 fixes K = KT at compile time (the products then run as straight-line
// code, with no loop-carried loads in flight); KT = 0 takes K at run time.
template <int LOGV, int KT>
__global__ void __launch_bounds__(FftShape<LOGV>::TPB) k_fft_sub_inv(Dev p, int rd, const float4 *__restrict__ scratch,
                                                                     const float4 *__restrict__ spec, int Kr,
                                                                     int o0, int nO, long long nfix, int advance) {
    using S = FftShape<LOGV>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int lt = threadIdx.x;
    const int K = KT > 0 ? KT : Kr;
    const long long U = (long long)K * N;
    const long long n = nfix > 0 ? nfix : position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    long long tile;
    int o;
    xcd_tile(blockIdx.x, (long long)p.M * p.B * p.D, nO, tile, o);
    // uniform: kept in scalar registers, so the loads below take scalar bases
    tile = __builtin_amdgcn_readfirstlane((int)tile);
    o = __builtin_amdgcn_readfirstlane(o + o0);
    const int c = __builtin_amdgcn_readfirstlane((int)(tile % p.D));
    const int l = __builtin_amdgcn_readfirstlane((int)(tile / ((long long)p.D * p.B)));
    const size_t row = (size_t)tile * (size_t)p.L;
    float2 *adst = reinterpret_cast<float2 *>(p.buf + row + t + 1 + (long long)o * N);
    const float4 *A = scratch + (size_t)tile * K * (N / 2);
    const float4 *G = spec + ((size_t)l * p.D + c) * (size_t)(2 * K - 1) * (N / 2);
    float2 *X = smem;
    // Z = sum_i A_i * G_{K+o-i} for this thread's pairs, four pairs at a time:
    // chunk q (pairs q*CH .. q*CH+CH-1) runs the K sub-blocks in steps
    // s = q*K + i.  The loads of step s + 1 are in flight while step s
    // multiplies; the prefetch is issued every time (the last one repeats the
    // final step's loads), so that the wait before each step's products
    // leaves the next step's loads outstanding.  K is a power of two.
    constexpr int PAIRS = (N / 2 + TT - 1) / TT;
    constexpr int CH = 4, NCH = PAIRS / CH;
    static_assert(PAIRS % CH == 0, "pairs per thread");
    const int kl = __builtin_ctz((unsigned)K);
    const int steps = NCH * K;
    // buffer loads: a resource over the tile's bins and one over the row's
    // offset spectra, the step's offset in a scalar register and one lane
    // offset, so no load needs vector address arithmetic
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)A, 0, (int)((size_t)K * (N / 2) * sizeof(float4)), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(
        (void *)G, 0, (int)((size_t)(2 * K - 1) * (N / 2) * sizeof(float4)), kBufferWord3);
    const unsigned vo = (unsigned)lt * (unsigned)sizeof(float4);
    auto load = [&](int st, float4(&a)[CH], float4(&g)[CH]) {
        const int i = st & (K - 1);
        const int off = (st >> kl) * CH * TT;
        const int sa = (i * (N / 2) + off) * (int)sizeof(float4);
        const int sg = ((K + o - i - 1) * (N / 2) + off) * (int)sizeof(float4);
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            a[m] = buffer_load4(rA, vo, sa + m * TT * (int)sizeof(float4));
            g[m] = buffer_load4(rG, vo, sg + m * TT * (int)sizeof(float4));
        }
    };
    float4 Z[CH];
    auto mac = [&](int q, const float4(&a)[CH], const float4(&g)[CH]) {
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            if (lt + (q * CH + m) * TT == 0) {  // (G_0, G_N) real, G_{N/2} complex
                Z[m].x = fmaf(a[m].x, g[m].x, Z[m].x);
                Z[m].y = fmaf(a[m].y, g[m].y, Z[m].y);
                const float2 h = cmul(make_float2(a[m].z, a[m].w), make_float2(g[m].z, g[m].w));
                Z[m].z += h.x;
                Z[m].w += h.y;
            } else {
                const float2 z1 = cmul(make_float2(a[m].x, a[m].y), make_float2(g[m].x, g[m].y));
                const float2 z2 = cmul(make_float2(a[m].z, a[m].w), make_float2(g[m].z, g[m].w));
                Z[m] = make_float4(Z[m].x + z1.x, Z[m].y + z1.y, Z[m].z + z2.x, Z[m].w + z2.y);
            }
        }
    };
    const PairLds pl = pair_lds<LOGV>(lt);
    float4 a0[CH], g0[CH], a1[CH], g1[CH];
    load(0, a0, g0);
    static_for<0, NCH>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        // this chunk's pair twiddles for the re-packing, read with its first
        // loads, so that no wait on them drains the step loads in flight
        float2 wc[CH];
#pragma unroll
        for (int m = 0; m < CH; ++m) wc[m] = p.ptw[N / 2 + lt + (q * CH + m) * TT];
#pragma unroll
        for (int m = 0; m < CH; ++m) Z[m] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < K; i += 2) {
            const int st = q * K + i;
            load(st + 1, a1, g1);
            mac(q, a0, g0);
            // each prefetch lands in the registers the products before it have
            // just read: the empty statement takes the sums as operands and
            // orders memory, so no load is hoisted above the products that free
            // its registers (hoisted, the loads need registers of their own and
            // spill)
            hold_after(Z);
            load(st + 2 < steps ? st + 2 : st + 1, a0, g0);
            mac(q, a1, g1);
            hold_after(Z);
        }
        // re-pack the finished chunk for the inverse transform
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            const int j = lt + (q * CH + m) * TT;
            if (j == 0) {
                const float Z0 = Z[m].x, ZN = Z[m].y;
                X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
                X[lpad(1)] = make_float2(Z[m].z, -Z[m].w);
            } else {
                const SlotPair sl = item_lds<LOGV, TT>(pl, lt, q * CH + m);
                float2 D1, D2;
                pack_inverse(make_float2(Z[m].x, Z[m].y), make_float2(Z[m].z, Z[m].w), wc[m], D1, D2);
                X[sl.a] = D1;
                X[sl.b] = D2;
            }
        }
    });
    const float2 wi = group_root<LOGV, S::NPASS - 1>(lt, p.twid, p.logNT);
    __syncthreads();
    const float2 w0 = inverse_groups<LOGV, S::NPASS - 1>(X, lt, p.twid, p.logNT, wi);
    // the pending sums of the output sub-block, read during the last group
    float2 acc[HALF0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) acc[m] = adst[lt + (m << QLOG0)];
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt) + lpad_off(m, QLOG0)];
    dit_group_w<R0>(v, w0);
#pragma unroll
    for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    finish_position(p, n, advance);
}


}  // namespace fi
