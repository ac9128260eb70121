// Kernels of the data-dependent-filter path: the filter taps arrive with the
// data, one per position, so both factors of every product are online.
//
// Flash Inference (arXiv 2410.12982), summary page, "Datenabhaengige
// Filter-Erweiterung (Appendix B)": a modified tiling (Algorithm 5) handles a
// filter that depends on the data at twice the work; each block then runs two
// same-size transforms instead of one.  The tiling used here (position n
// 0-based, p a power of two):
//   red cell     y_n = pend_n + x_n h_0 + x_0 h_n            (x_0 h_0 at n = 0)
//   square       x[p, 2p) * h[p, 2p)                          at n = 2p - 1
//   band blocks  x[n+1-p, n+1) * h[p, 2p) and
//                h[n+1-p, n+1) * x[p, 2p)                     at n = (m+1)p - 1, m >= 2
// Every pair (i, j) of x_i h_j is formed once, at a position where both are
// known and before its target i + j.  A product of two p-blocks adds into the
// 2p - 1 targets from n + 1 on; small p directly, large p as one 2p-point
// circular convolution per product (no wrap: the linear length is 2p - 1)
// against the cached spectrum of the fixed block x[p, 2p) or h[p, 2p).
//
// Storage per row r = b*D + c: xh[r][L], hh[r][L] the inputs and taps so far,
// acc[r][L] the pending sums; per FFT size p, spx/sph[r][p/2] float4 the
// spectra of x[p, 2p) and h[p, 2p) (pair order, scaled by 1/p).
#pragma once
#include "fi_device.h"
#include "fi_fft.h"
#include "fi_fft_kernels.h"

namespace fi {

struct DDev {
    float *xh, *hh, *acc;
    long long L;
    int R;          // rows B * D
    int pd;         // products of blocks p < pd run directly
};

// Direct products run in one launch per position up to this block size; wider
// direct products (only when the FFT threshold is set above it) take the
// serial per-row loop below.
constexpr int kDDNearMax = 128;

// Red cells of position n and every direct product of that position with
// p <= PM.  The products of a position are those of p = 1, 2, 4, .., pm (each
// condition on p -- below the FFT threshold, 2p <= n + 1, p | n + 1 -- holds
// for all smaller powers of two once it holds for pm), so the host passes the
// largest one as PM (prod false: no products, red cells only).  2 PM threads
// per row, thread j owns target n + 1 + j (j < 2 PM - 1) and sums its terms of
// every size at once; thread 0 also forms the red cell.  Per row, LDS holds
// x and h over [0, 2 PM) (the fixed blocks [p, 2p)) and over (n - PM, n] (the
// newest blocks), with position n taken from the arriving x_n, h_n.
template <int PM>
__global__ void __launch_bounds__(256) k_dd_near(DDev q, long long n, const float *__restrict__ x,
                                                 const float *__restrict__ h, float *__restrict__ y, bool prod) {
    constexpr int TR = 2 * PM, RPW = 256 / TR;
    __shared__ float fx[RPW][TR], fh[RPW][TR], nx[RPW][PM], nh[RPW][PM];
    const int lr = threadIdx.x / TR, j = threadIdx.x % TR;
    const int r = blockIdx.x * RPW + lr;
    const bool live = r < q.R;
    const size_t base = (size_t)(live ? r : 0) * q.L;
    const float *xr = q.xh + base, *hr = q.hh + base;
    float xn = 0.f, hn = 0.f;
    if (live) {
        xn = x[r];
        hn = h[r];
    }
    if (prod && live) {
        // every index read here is <= n, since 2 PM <= n + 1
        fx[lr][j] = j == n ? xn : xr[j];
        fh[lr][j] = j == n ? hn : hr[j];
        if (j < PM) {
            const long long i = n + 1 - PM + j;
            nx[lr][j] = i == n ? xn : xr[i];
            nh[lr][j] = i == n ? hn : hr[i];
        }
    }
    if (live && j == 0) {
        float *ar = q.acc + base;
        q.xh[base + n] = xn;
        q.hh[base + n] = hn;
        y[r] = n == 0 ? xn * hn : fmaf(xr[0], hn, fmaf(xn, hr[0], ar[n]));
    }
    if (!prod) return;
    __syncthreads();
    if (!live || j >= TR - 1 || n + 1 + j >= q.L) return;
    // term (a, b): newest-block element a times fixed-block element b, a + b = j.
    // b runs over the whole block (compile-time trip counts, so the LDS reads
    // pipeline); a = j - b outside [0, p) leaves the sums as they are.
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int p = 1; p <= PM; p *= 2) {
        if (j >= 2 * p - 1) continue;
        const bool square = n + 1 == 2 * p;
#pragma unroll
        for (int b = 0; b < p; ++b) {
            const int a = j - b;
            const bool ok = (unsigned)a < (unsigned)p;
            const int ai = PM - p + (ok ? a : 0);
            const float s1 = fmaf(nx[lr][ai], fh[lr][p + b], s), t1 = fmaf(nh[lr][ai], fx[lr][p + b], t);
            s = ok ? s1 : s;
            t = ok && !square ? t1 : t;
        }
    }
    s += t;
    q.acc[base + n + 1 + j] += s;
}

// Red cells of position n for a stack of M data-dependent layers, one thread
// per (b, c) chain through every layer (rows r = l * BD + b * D + c): layer
// l's input x (layer 0: x0, the arriving input; layer l+1: tanh of layer l's
// output), its arriving tap h[r], its pending sum and first input and tap.
// Each layer's input goes to xs[r] for the position's product kernels, which
// store x_n, h_n and form the same red cell again (the same operations on the
// same values, so y is written twice with one value).
static __global__ void __launch_bounds__(256) k_dd_chain(DDev q, int M, int BD, long long n,
                                                         const float *__restrict__ x0, const float *__restrict__ h,
                                                         float *__restrict__ y, float *__restrict__ xs) {
    const int bc = blockIdx.x * 256 + threadIdx.x;
    if (bc >= BD) return;
    float x = x0[bc];
    for (int l = 0; l < M; ++l) {
        const int r = l * BD + bc;
        const size_t base = (size_t)r * q.L;
        const float hn = h[r];
        xs[r] = x;
        const float yl = n == 0 ? x * hn : fmaf(q.xh[base], hn, fmaf(x, q.hh[base], q.acc[base + n]));
        y[r] = yl;
        x = tanhf(yl);
    }
}

// Direct products of kDDNearMax < p < pd at position n, one thread per row,
// after k_dd_near (which stored x_n, h_n).  Both products of a band block go
// to the same targets.
static __global__ void __launch_bounds__(256) k_dd_wide(DDev q, long long n) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= q.R) return;
    const float *xr = q.xh + (size_t)r * q.L, *hr = q.hh + (size_t)r * q.L;
    float *ar = q.acc + (size_t)r * q.L;
    for (long long p = 2 * kDDNearMax; p < q.pd && 2 * p <= n + 1 && (n + 1) % p == 0; p *= 2) {
        const bool square = n + 1 == 2 * p;
        const long long lo = n + 1 - p;           // newest block [lo, n]
        for (long long j = 0; j < 2 * p - 1 && n + 1 + j < q.L; ++j) {
            float s = 0.f;
            const long long a0 = j < p ? 0 : j - p + 1, a1 = j < p ? j : p - 1;
            for (long long a = a0; a <= a1; ++a) {
                s = fmaf(xr[lo + a], hr[p + j - a], s);
                if (!square) s = fmaf(hr[lo + a], xr[p + j - a], s);
            }
            ar[n + 1 + j] += s;
        }
    }
}

// Spectra of the fixed blocks x[p, 2p) and h[p, 2p) (p = 2^LOGN complex
// points carry the 2p-point real transform of the zero-padded block), in
// pair order, scaled by 1/p.  One team per row; blockIdx.y: 0 x, 1 h.
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) __attribute__((amdgpu_waves_per_eu(LOGN >= 8 ? 4 : 1)))
k_dd_band(Dev p, DDev q, float4 *__restrict__ spx, float4 *__restrict__ sph) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long row = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = row < q.R;
    const long long rr = active ? row : 0;
    float2 *X = smem + team * lds_len(N);
    const float *base = (blockIdx.y == 0 ? q.xh : q.hh) + (size_t)rr * q.L + N;
    const float2 *src = reinterpret_cast<const float2 *>(base);
    float4 *dst = (blockIdx.y == 0 ? spx : sph) + (size_t)rr * (N / 2);
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) {
        v[m] = active ? src[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
        v[m + HALF0] = make_float2(0.f, 0.f);
    }
    dif_group<R0, true>(v, lt, LOGN, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt) + lpad_off(m, QLOG0)] = v[m];
    forward_groups<LOGN, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    if (!active) return;
    const float inv = 1.0f / (float)N;
    for (int e = lt; e < N / 2; e += TT) {
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

// The FFT products of position n for block size p = 2^LOGN (n + 1 a multiple
// of p): the square x[p, 2p) * h[p, 2p) when n + 1 = 2p, else both band
// products; all 2p - 1 targets from n + 1 on (below L) take the sum.
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) __attribute__((amdgpu_waves_per_eu(LOGN >= 8 ? 4 : 1)))
k_dd_fft(Dev p, DDev q, const float4 *__restrict__ spx, const float4 *__restrict__ sph, long long n) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long row = (long long)blockIdx.x * S::PER_BLOCK + team;
    const bool active = row < q.R;
    const long long rr = active ? row : 0;
    float2 *X = smem + team * lds_len(N);
    const bool square = n + 1 == 2 * N;
    const long long lo = n + 1 - N;
    const float *xr = q.xh + (size_t)rr * q.L, *hr = q.hh + (size_t)rr * q.L;
    float2 va[1 << R0], vb[1 << R0];
    // x[lo, n] against the spectrum of h[p, 2p)
    fft_block<LOGN, false>(p, X, lt, active, reinterpret_cast<const float2 *>(xr + lo), sph + (size_t)rr * (N / 2), va,
                    []() {});
    if (!square) {
        __syncthreads();  // the second transform reuses the LDS
        fft_block<LOGN, false>(p, X, lt, active, reinterpret_cast<const float2 *>(hr + lo), spx + (size_t)rr * (N / 2),
                        vb, []() {});
    }
    if (!active) return;
    float *ar = q.acc + (size_t)rr * q.L + n + 1;
    const long long room = q.L - (n + 1);     // targets below L
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) {
        const long long g = lt + ((long long)m << QLOG0);   // output pair 2g, 2g + 1
        float2 s = va[m];
        if (!square) s = cadd(s, vb[m]);
        if (2 * g < room) ar[2 * g] += s.x;
        if (2 * g + 1 < room && 2 * g + 1 < 2 * N - 1) ar[2 * g + 1] += s.y;
    }
}

}  // namespace fi
