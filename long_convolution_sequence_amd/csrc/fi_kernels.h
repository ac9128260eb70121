// Kernels of one position ("step") of the relaxed schedule.
//
// Flash Inference (arXiv 2410.12982), summary page:
//  * red cell (Algorithm 1/2): y^l_n = (pending sum at n) + h^l[c][0] * x^l_n;
//  * gray block after n, U = largest power of two dividing n:
//    outputs n+1..n+U receive sum_{s=n-U+1..n} h^l[c][t-s] x^l_s;
//  * Algorithm 3: red cells run layer after layer, the gray blocks of all
//    layers have no mutual dependence and run in one launch.
// Positions are 1-based (n); activation slots are 0-based (t = n-1).
#pragma once
#include "fi_device.h"
#include "fi_fft.h"

namespace fi {

// ---------------------------------------------------------------------------
// Red cells of one (b, c) chain through all layers at position n.
// Reads the pending sums, writes the layer inputs into their slots (the slot
// of position n switches from "pending sum" to "input"), the recorded y, the
// last output and the next feedback input.  xs (optional) receives x^l_n.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float chain_input(const Dev &p, long long n, int chain, const float *xext) {
    const int BD = p.B * p.D;
    return xext ? xext[chain] : p.xin[(size_t)(n & 1) * BD + chain];
}

__device__ __forceinline__ void chain_output(const Dev &p, long long n, int chain, float ylast, float *yext) {
    const int BD = p.B * p.D;
    const long long t = n - 1;
    p.ylast[(size_t)t * BD + chain] = ylast;
    if (yext) yext[chain] = ylast;
    p.xin[(size_t)((n + 1) & 1) * BD + chain] = apply_map(p.fb, ylast);
}

// Red cells for every chain; one thread per (b, c).  `advance` is set when no
// other kernel of this position follows.
__global__ void __launch_bounds__(256) k_red(Dev p, const float *xext, float *yext, int advance) {
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L) return;  // uniform: never touch memory past position L
    const int chain = blockIdx.x * blockDim.x + threadIdx.x;
    if (chain < p.B * p.D) {
        const int b = chain / p.D, c = chain % p.D;
        float x = chain_input(p, n, chain, xext);
        float y = 0.f;
        constexpr int CHUNK = 16;
        for (int l0 = 0; l0 < p.M; l0 += CHUNK) {
            float pend[CHUNK], h0[CHUNK];
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) {
                if (l0 + i < p.M) {
                    pend[i] = p.buf[act_row(p, l0 + i, b, c) + t];
                    h0[i] = p.filt[filt_row(p, l0 + i, c)];
                }
            }
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) {
                if (l0 + i < p.M) {
                    const int l = l0 + i;
                    const size_t r = act_row(p, l, b, c) + t;
                    y = fmaf(h0[i], x, pend[i]);
                    p.buf[r] = x;
                    if (p.rec) p.rec[r] = y;
                    x = apply_map(p.map, y);
                }
            }
        }
        chain_output(p, n, chain, y, yext);
    }
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// One position whose gray block is computed directly, fused with the red
// cells: a workgroup owns CH whole chains (all layers), so the slot written by
// a red cell is read by tiles of the same workgroup only.
//   phase 0: every thread prefetches pending sums, h0, the input window,
//            the taps h[1..2U-1] and the U pending outputs into LDS;
//   phase 1: one thread per chain runs the red cells through the layers;
//   phase 2: one thread per output adds the U-term dot product.
// CHAIN = false: the layer inputs at n are already in their slots (external
// block mode); phase 1 is skipped.
// ---------------------------------------------------------------------------
template <int U, bool CHAIN>
__global__ void __launch_bounds__(256) k_step_direct(Dev p, int CH, const float *xext, float *yext,
                                                     int advance) {
    extern __shared__ float sm[];
    const int M = p.M;
    const int items = M * CH;
    float *pend = sm;                    // [M*CH]
    float *h0 = pend + items;            // [M*CH]
    float *xw = h0 + items;              // [M*CH][U]   inputs at n-U+1..n
    float *tp = xw + items * U;          // [M*CH][2U-1] taps h[1..2U-1]
    float *aw = tp + items * (2 * U - 1);  // [M*CH][U] pending sums at n+1..n+U

    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    // uniform guard: a gray block of edge U exists only after multiples of U
    // and ends at or before L; any other position is left untouched
    if (n > p.L || n % U != 0 || n + U > p.L) return;
    const int BD = p.B * p.D;
    const int ch0 = blockIdx.x * CH;
    const int nch = min(CH, BD - ch0);
    const int tid = threadIdx.x, bs = blockDim.x;

    for (int i = tid; i < items; i += bs) {
        const int l = i / CH, k = i % CH;
        if (k < nch) {
            const int chain = ch0 + k, b = chain / p.D, c = chain % p.D;
            if (CHAIN) pend[i] = p.buf[act_row(p, l, b, c) + t];
            h0[i] = p.filt[filt_row(p, l, c)];
        }
    }
    constexpr int XW = CHAIN ? U - 1 : U;  // window entries read from memory
    if constexpr (XW > 0) {
        for (int i = tid; i < items * XW; i += bs) {
            const int lk = i / XW, kk = i % XW;
            const int l = lk / CH, k = lk % CH;
            if (k < nch) {
                const int chain = ch0 + k, b = chain / p.D, c = chain % p.D;
                xw[lk * U + kk] = p.buf[act_row(p, l, b, c) + t - (U - 1) + kk];
            }
        }
    }
    for (int i = tid; i < items * (2 * U - 1); i += bs) {
        const int lk = i / (2 * U - 1), m = i % (2 * U - 1);
        const int l = lk / CH, k = lk % CH;
        if (k < nch) {
            const int c = (ch0 + k) % p.D;
            tp[i] = p.filt[filt_row(p, l, c) + 1 + m];
        }
    }
    for (int i = tid; i < items * U; i += bs) {
        const int lk = i / U, j = i % U;
        const int l = lk / CH, k = lk % CH;
        if (k < nch) {
            const int chain = ch0 + k, b = chain / p.D, c = chain % p.D;
            aw[i] = p.buf[act_row(p, l, b, c) + t + 1 + j];
        }
    }
    __syncthreads();

    if (CHAIN && tid < nch) {
        const int chain = ch0 + tid, b = chain / p.D, c = chain % p.D;
        float x = chain_input(p, n, chain, xext);
        float y = 0.f;
        for (int l = 0; l < M; ++l) {
            const int i = l * CH + tid;
            const size_t r = act_row(p, l, b, c) + t;
            y = fmaf(h0[i], x, pend[i]);
            p.buf[r] = x;
            if (p.rec) p.rec[r] = y;
            xw[i * U + (U - 1)] = x;
            x = apply_map(p.map, y);
        }
        chain_output(p, n, chain, y, yext);
    }
    __syncthreads();

    for (int i = tid; i < items * U; i += bs) {
        const int lk = i / U, j = i % U;
        const int l = lk / CH, k = lk % CH;
        if (k < nch) {
            const int chain = ch0 + k, b = chain / p.D, c = chain % p.D;
            const float *x = xw + lk * U;
            const float *h = tp + lk * (2 * U - 1) + j + U - 1;   // h[j+U-kk] = h[-kk]
            float s = aw[i];
#pragma unroll
            for (int kk = 0; kk < U; ++kk) s = fmaf(h[-kk], x[kk], s);
            p.buf[act_row(p, l, b, c) + t + 1 + j] = s;
        }
    }
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// Gray blocks of all layers by FFT, U = 2^LOGN (complex transform of U points
// carries the 2U-point real circular convolution).  One team of TT threads per
// (l, b, c) block; the red cells at n have already run.
//   spec: per (l, c), U/2 float4 in pair order (see k_spectrum), scaled by 1/U.
// ---------------------------------------------------------------------------
template <int LOGN>
__global__ void __launch_bounds__(FftShape<LOGN>::TPB) k_fft_tile(Dev p, const float4 *__restrict__ spec,
                                                                  int advance) {
    using S = FftShape<LOGN>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int team = threadIdx.x / TT, lt = threadIdx.x % TT;
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L || n % N != 0 || n + N > p.L) return;  // uniform guard, as in k_step_direct
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

    float2 acc[HALF0];
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) {
        acc[m] = active ? adst[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
        v[m] = active ? xsrc[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
        v[m + HALF0] = make_float2(0.f, 0.f);
    }
    dif_group<R0, true>(v, lt, LOGN, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGN, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();

    // bins of the real transform times the filter spectrum, re-packed for the inverse
    for (int j = lt; j < N / 2; j += TT) {
        const float4 g = active ? sp[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (j == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            const float Z0 = (C0.x + C0.y) * g.x;
            const float ZN = (C0.x - C0.y) * g.y;
            X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
            X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w));
        } else {
            const int p1 = lpad(bitrev<LOGN>(j)), p2 = lpad(bitrev<LOGN>(N - j));
            const float2 W = twiddle(p.twid, p.logNT, LOGN + 1, j);
            float2 A1, A2, D1, D2;
            real_bins(X[p1], X[p2], W, A1, A2);
            pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2);
            X[p1] = D1;
            X[p2] = D2;
        }
    }
    __syncthreads();
    inverse_groups<LOGN, S::NPASS - 1>(X, lt, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
    dit_group<R0>(v, lt, LOGN, p.twid, p.logNT);
    if (active) {
#pragma unroll
        for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    }
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// Filter spectra ("FFT-Vorberechnung"): for every (l, c) row, the 2N-point real
// FFT of the taps g_r = h[goff + r], r in [0, 2N), stored in pair order
//   spec[0] = (G_0, G_N, Re G_{N/2}, Im G_{N/2}) / N
//   spec[j] = (G_j, G_{N-j}) / N,  0 < j < N/2.
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
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGN, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    const float inv = 1.0f / (float)N;
    float4 *dst = spec + (size_t)rowi * (size_t)row_stride;
    for (int j = lt; j < N / 2 && active; j += TT) {
        if (j == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            dst[0] = make_float4((C0.x + C0.y) * inv, (C0.x - C0.y) * inv, Ch.x * inv, -Ch.y * inv);
        } else {
            float2 A1, A2;
            real_bins(X[lpad(bitrev<LOGN>(j))], X[lpad(bitrev<LOGN>(N - j))],
                      twiddle(p.twid, p.logNT, LOGN + 1, j), A1, A2);
            dst[j] = make_float4(A1.x * inv, A1.y * inv, A2.x * inv, A2.y * inv);
        }
    }
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
template <int LOGV>
__global__ void __launch_bounds__(FftShape<LOGV>::TPB) k_fft_sub_fwd(Dev p, float4 *__restrict__ scratch,
                                                                     int K) {
    using S = FftShape<LOGV>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    static_assert(S::PER_BLOCK == 1, "sub-block transforms fill a workgroup");
    __shared__ float2 smem[S::LDS];
    const int lt = threadIdx.x;
    const long long U = (long long)K * N;
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    const long long tile = (long long)blockIdx.x / K;
    const int i = (int)(blockIdx.x % K);
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
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGV, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    float4 *dst = scratch + ((size_t)tile * K + i) * (N / 2);
    for (int j = lt; j < N / 2; j += TT) {
        if (j == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            dst[0] = make_float4(C0.x + C0.y, C0.x - C0.y, Ch.x, -Ch.y);
        } else {
            float2 A1, A2;
            real_bins(X[lpad(bitrev<LOGV>(j))], X[lpad(bitrev<LOGV>(N - j))],
                      twiddle(p.twid, p.logNT, LOGV + 1, j), A1, A2);
            dst[j] = make_float4(A1.x, A1.y, A2.x, A2.y);
        }
    }
}

// k_fft_sub_inv: per (l, b, c, o), Z = sum_i A_i * G_{K+o-i}, then the inverse
// transform and accumulation of its exact upper half into output sub-block o.
template <int LOGV>
__global__ void __launch_bounds__(FftShape<LOGV>::TPB) k_fft_sub_inv(Dev p, const float4 *__restrict__ scratch,
                                                                     const float4 *__restrict__ spec, int K,
                                                                     int advance) {
    using S = FftShape<LOGV>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int lt = threadIdx.x;
    const long long U = (long long)K * N;
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    const long long tile = (long long)blockIdx.x / K;
    const int o = (int)(blockIdx.x % K);
    const int c = (int)(tile % p.D);
    const int l = (int)(tile / ((long long)p.D * p.B));
    const size_t row = (size_t)tile * (size_t)p.L;
    float2 *adst = reinterpret_cast<float2 *>(p.buf + row + t + 1 + (long long)o * N);
    const float4 *A = scratch + (size_t)tile * K * (N / 2);
    const float4 *G = spec + ((size_t)l * p.D + c) * (size_t)(2 * K - 1) * (N / 2);
    float2 *X = smem;
    float2 acc[HALF0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) acc[m] = adst[lt + (m << QLOG0)];
    for (int j = lt; j < N / 2; j += TT) {
        if (j == 0) {
            float Z0 = 0.f, ZN = 0.f;
            float2 Zh = make_float2(0.f, 0.f);
            for (int i = 0; i < K; ++i) {
                const float4 a = A[(size_t)i * (N / 2)];
                const float4 g = G[(size_t)(K + o - i - 1) * (N / 2)];
                Z0 = fmaf(a.x, g.x, Z0);
                ZN = fmaf(a.y, g.y, ZN);
                Zh = cadd(Zh, cmul(make_float2(a.z, a.w), make_float2(g.z, g.w)));
            }
            X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
            X[lpad(1)] = make_float2(Zh.x, -Zh.y);
        } else {
            float2 Z1 = make_float2(0.f, 0.f), Z2 = make_float2(0.f, 0.f);
            for (int i = 0; i < K; ++i) {
                const float4 a = A[(size_t)i * (N / 2) + j];
                const float4 g = G[(size_t)(K + o - i - 1) * (N / 2) + j];
                Z1 = cadd(Z1, cmul(make_float2(a.x, a.y), make_float2(g.x, g.y)));
                Z2 = cadd(Z2, cmul(make_float2(a.z, a.w), make_float2(g.z, g.w)));
            }
            float2 D1, D2;
            pack_inverse(Z1, Z2, twiddle(p.twid, p.logNT, LOGV + 1, j), D1, D2);
            X[lpad(bitrev<LOGV>(j))] = D1;
            X[lpad(bitrev<LOGV>(N - j))] = D2;
        }
    }
    __syncthreads();
    inverse_groups<LOGV, S::NPASS - 1>(X, lt, p.twid, p.logNT);
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
    dit_group<R0>(v, lt, LOGV, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// Lazy baseline, sum part: for every (l, b, c), the pending sum at n is the
// whole history term sum_{s=1..n-1} h[n-s] x_s, written into slot n-1; the
// red cells (k_red) then add h[0] x_n.  One workgroup per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_lazy_dot(Dev p) {
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L) return;
    const long long rowi = blockIdx.x;
    const int b = (int)((rowi / p.D) % p.B), c = (int)(rowi % p.D);
    const int l = (int)(rowi / ((long long)p.D * p.B));
    const float *x = p.buf + act_row(p, l, b, c);
    const float *h = p.filt + filt_row(p, l, c);
    float s = 0.f;
    for (long long k = threadIdx.x; k < t; k += blockDim.x) s = fmaf(h[t - k], x[k], s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.f;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += part[w];
        p.buf[act_row(p, l, b, c) + t] = tot;
    }
}

// ---------------------------------------------------------------------------
// External-block mode: the red cell of one layer at position n for all (b, c):
// y = pending + h0 * q, and q becomes the slot's input.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_red_layer(Dev p, int l, const float *q, float *y) {
    const long long n = p.st->pos + 1;
    const long long t = n - 1;
    if (n > p.L) return;
    const int chain = blockIdx.x * blockDim.x + threadIdx.x;
    if (chain < p.B * p.D) {
        const int b = chain / p.D, c = chain % p.D;
        const size_t r = act_row(p, l, b, c) + t;
        const float x = q[chain];
        const float v = fmaf(p.filt[filt_row(p, l, c)], x, p.buf[r]);
        p.buf[r] = x;
        if (p.rec) p.rec[r] = v;
        y[chain] = v;
        if (l == p.M - 1) p.ylast[(size_t)t * p.B * p.D + chain] = v;
    }
}

// Publish position n when no gray block follows (the last position, or
// external mode's last position).
__global__ void k_finish(Dev p) {
    if (p.st->pos + 1 > p.L) return;
    finish_position(p, p.st->pos + 1, 1);
}

}  // namespace fi
