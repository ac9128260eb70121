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

// Threads of a direct-block workgroup (one wave runs the red cells, the rest
// stage rows from memory: the staging is the critical path from U = 2 on, and
// sixteen waves measured 25-50% faster than four there) and of the
// ring <-> history copies at FFT positions.
constexpr int kDirectThreads = 1024;
constexpr int kRingThreads = 1024;

// ---------------------------------------------------------------------------
// Red cells of one (b, c) chain at position n, layers 0..l1-1, from the ring.
// The pending sum for (l, n) is final when position n starts; y^l_n adds the
// own-position term h^l[c][0] x^l_n and x^{l+1}_n = map(y^l_n).  Only layers
// l >= l0 are "owned" by the caller: their inputs go to the ring (and to xs,
// the caller's LDS copy, at stride xs_stride), the records, and (rowx) the
// row-major history.  The owner of the last layer also writes the output and
// the next feedback input.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void chain_output(const Dev &p, long long n, int chain, float ylast, float *yext) {
    const int BD = p.B * p.D;
    p.ylast[(size_t)(n - 1) * BD + chain] = ylast;
    if (yext) yext[chain] = ylast;
    p.xin[(size_t)((n + 1) & 1) * BD + chain] = apply_map(p.fb, ylast);
}

__device__ __forceinline__ void run_chain(const Dev &p, long long n, int chain, int l0, int l1,
                                          const float *xext, float *yext, float *xs, int xs_stride, bool rowx) {
    const int BD = p.B * p.D;
    const int b = chain / p.D, c = chain % p.D;
    float x = xext ? xext[chain] : p.xin[(size_t)(n & 1) * BD + chain];
    float y = 0.f;
    constexpr int CHUNK = 24;
    for (int lb = 0; lb < l1; lb += CHUNK) {
        float pend[CHUNK], h0[CHUNK];
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) {
            if (lb + i < l1) {
                pend[i] = p.ar[ring(p, n, lb + i) + chain];
                h0[i] = p.hh[head(p, lb + i, 0, c)];
            }
        }
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) {
            const int l = lb + i;
            if (l < l1) {
                y = fmaf(h0[i], x, pend[i]);
                if (l >= l0) {
                    p.xr[ring(p, n, l) + chain] = x;
                    if (xs) xs[(l - l0) * xs_stride] = x;
                    if (p.recx) {
                        const size_t r = ((size_t)(n - 1) * p.M + l) * BD + chain;
                        p.recx[r] = x;
                        p.recy[r] = y;
                    }
                    if (rowx) p.buf[act_row(p, l, b, c) + (n - 1)] = x;
                }
                x = apply_map(p.map, y);
            }
        }
    }
    if (l1 == p.M) chain_output(p, n, chain, y, yext);
}

// The ring slot of position n + W/2 is reused by that position: clear it for
// the owned layers.  Nothing reads or adds to it during position n (pending
// sums only ever target positions n+1 .. n+W/2-1 before the drain, which runs
// after this kernel).
__device__ __forceinline__ void clear_ahead(const Dev &p, long long n, int chain, int l0, int l1, int wave,
                                            int waves) {
    for (int l = l0 + wave; l < l1; l += waves) p.ar[ring(p, n + p.W / 2, l) + chain] = 0.f;
}

// ---------------------------------------------------------------------------
// One position whose gray block (edge U) is computed directly, fused with the
// red cells.  Block = 64 chains (lanes) x 4 waves, grid = chain blocks x layer
// groups of LG layers.  Each block recomputes the red cells of its chains up to
// its last layer (cheap, and no other block can be waited on) but writes only
// its own layers.  The gray block is a U x U Toeplitz product per chain:
//   pending(n+1+j) += sum_k h[j+U-k] x_{n-U+1+k},  j, k in [0, U)
// with inputs and taps staged in LDS and a sliding register window of J taps.
// U = 0: red cells only (the last position).  CHAIN = false: the layer inputs
// at n are already in the ring (external block mode).
// ---------------------------------------------------------------------------
template <int U, bool CHAIN>
__global__ void __launch_bounds__(kDirectThreads) k_direct(Dev p, int rd, int LG, const float *xext, float *yext,
                                                int advance, int rowx) {
    extern __shared__ float sm[];
    const long long n = position_of(p, rd);
    if (n > p.L) return;  // uniform guards: never touch memory past position L
    if constexpr (U > 0) {
        if (n % U != 0 || n + U > p.L) return;
    }
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x / kLanes;
    const int BD = p.B * p.D;
    const int cb = blockIdx.x * kLanes;
    const int chain = cb + lane;
    const bool live = chain < BD;
    const int l0 = blockIdx.y * LG, l1 = min(p.M, l0 + LG), nl = l1 - l0;
    if constexpr (U == 0) {
        if (wave == 0 && CHAIN && live) run_chain(p, n, chain, l0, l1, xext, yext, nullptr, 0, rowx != 0);
        if (live) clear_ahead(p, n, chain, l0, l1, wave, blockDim.x / kLanes);
    } else {
        constexpr int TAPS = 2 * U - 1;
        float *xw = sm;                               // [LG][U][64]: inputs at n-U+1 .. n
        float *tp = xw + (size_t)LG * U * kLanes;     // [LG][2U-1][64]: taps h[1 .. 2U-1]
        float *aw = tp + (size_t)LG * TAPS * kLanes;  // [LG][U][64]: pending sums at n+1 .. n+U
        if (wave == 0) {
            // wave 0: the red cells (its loads are the first it issues)
            if (CHAIN && live)
                run_chain(p, n, chain, l0, l1, xext, yext, xw + (U - 1) * kLanes + lane, U * kLanes, rowx != 0);
        } else {
            // waves 1..: stage the input window, the taps and the pending outputs
            // (eight loads in flight per thread: fewer measured slower, more too)
            const int t2 = threadIdx.x - kLanes, b2 = blockDim.x - kLanes;
            constexpr int KW = CHAIN ? U - 1 : U;     // window entries taken from the ring
            constexpr int KD = KW > 0 ? KW : 1;       // divisor (no entries when KW is 0)
            batched_copy<8>(nl * KW * kLanes, t2, b2,
                [&](int i) {
                    const int ln = i & (kLanes - 1), k = (i / kLanes) % KD, li = (i / kLanes) / KD;
                    return cb + ln < BD ? p.xr[ring(p, n - U + 1 + k, l0 + li) + cb + ln] : 0.f;
                },
                [&](int i, float v) {
                    const int ln = i & (kLanes - 1), k = (i / kLanes) % KD, li = (i / kLanes) / KD;
                    xw[(li * U + k) * kLanes + ln] = v;
                });
            batched_copy<8>(nl * TAPS * kLanes, t2, b2,
                [&](int i) {
                    const int ln = i & (kLanes - 1), m = (i / kLanes) % TAPS, li = (i / kLanes) / TAPS;
                    return cb + ln < BD ? p.hh[head(p, l0 + li, 1 + m, (cb + ln) % p.D)] : 0.f;
                },
                [&](int i, float v) { tp[i] = v; });
            batched_copy<8>(nl * U * kLanes, t2, b2,
                [&](int i) {
                    const int ln = i & (kLanes - 1), j = (i / kLanes) % U, li = (i / kLanes) / U;
                    return cb + ln < BD ? p.ar[ring(p, n + 1 + j, l0 + li) + cb + ln] : 0.f;
                },
                [&](int i, float v) { aw[i] = v; });
            if (live) clear_ahead(p, n, chain, l0, l1, wave - 1, blockDim.x / kLanes - 1);
        }
        __syncthreads();
        constexpr int J = U < 8 ? U : 8;              // outputs per task
        constexpr int NJ = U / J;
        if (live) {
            for (int task = wave; task < nl * NJ; task += blockDim.x / kLanes) {
                const int li = task / NJ, j0 = (task % NJ) * J;
                const float *x = xw + (size_t)li * U * kLanes + lane;
                const float *h = tp + (size_t)li * TAPS * kLanes + lane;   // h[m*64] = tap m+1
                const float *a = aw + (size_t)li * U * kLanes + lane;
                float acc[J], hw[J];
#pragma unroll
                for (int jj = 0; jj < J; ++jj) {
                    acc[jj] = a[(j0 + jj) * kLanes];
                    hw[jj] = h[(j0 + jj + U - 1) * kLanes];                // tap index for k = 0
                }
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const float xv = x[k * kLanes];
#pragma unroll
                    for (int jj = 0; jj < J; ++jj) acc[jj] = fmaf(hw[jj], xv, acc[jj]);
                    if (k + 1 < U) {                                        // slide: tap index - 1
#pragma unroll
                        for (int jj = J - 1; jj > 0; --jj) hw[jj] = hw[jj - 1];
                        hw[0] = h[(j0 + U - k - 2) * kLanes];
                    }
                }
#pragma unroll
                for (int jj = 0; jj < J; ++jj) p.ar[ring(p, n + 1 + j0 + jj, l0 + li) + chain] = acc[jj];
            }
        }
    }
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// First kernel of a position with an FFT gray block (n a multiple of G): the
// red cells, then the inputs of positions n-G+1 .. n of every owned row are
// copied from the ring into the row-major history (through an LDS transpose so
// both sides are coalesced).  CHAIN = false: external block mode.
// ---------------------------------------------------------------------------
template <bool CHAIN>
__global__ void __launch_bounds__(kRingThreads) k_red_fft(Dev p, int rd, int LG, const float *xext, float *yext) {
    extern __shared__ float sm[];                 // [LG][G][65]
    const long long n = position_of(p, rd);
    const int G = p.G;
    if (n > p.L || G < 1 || n % G != 0) return;  // uniform guard
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x / kLanes;
    const int BD = p.B * p.D;
    const int cb = blockIdx.x * kLanes;
    const int chain = cb + lane;
    const bool live = chain < BD;
    const int l0 = blockIdx.y * LG, l1 = min(p.M, l0 + LG), nl = l1 - l0;
    constexpr int PAD = kLanes + 1;
    if (wave == 0) {
        if (CHAIN && live) run_chain(p, n, chain, l0, l1, xext, yext, sm + (G - 1) * PAD + lane, G * PAD, false);
    } else {
        const int KW = CHAIN ? G - 1 : G;
        batched_copy(nl * KW * kLanes, threadIdx.x - kLanes, blockDim.x - kLanes,
            [&](int i) {
                const int ln = i & (kLanes - 1), k = (i / kLanes) % KW, li = (i / kLanes) / KW;
                return cb + ln < BD ? p.xr[ring(p, n - G + 1 + k, l0 + li) + cb + ln] : 0.f;
            },
            [&](int i, float v) {
                const int ln = i & (kLanes - 1), k = (i / kLanes) % KW, li = (i / kLanes) / KW;
                sm[(li * G + k) * PAD + ln] = v;
            });
        if (live) clear_ahead(p, n, chain, l0, l1, wave - 1, blockDim.x / kLanes - 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nl * kLanes * G; i += blockDim.x) {
        const int k = i % G, ln = (i / G) % kLanes, li = (i / G) / kLanes;
        const int ch = cb + ln;
        if (ch < BD) p.buf[act_row(p, l0 + li, ch / p.D, ch % p.D) + (n - G) + k] = sm[(li * G + k) * PAD + ln];
    }
}

// Last kernel of an FFT position: the FFT gray blocks' pending sums for
// positions n+1 .. n+G are final (the next FFT block starts at n+G); add them
// from the row-major history into the ring.  Grid = chain blocks x layers.
__global__ void __launch_bounds__(kRingThreads) k_drain(Dev p, int rd, int advance) {
    extern __shared__ float sm[];                 // [G][65]
    const long long n = position_of(p, rd);
    const int G = p.G;
    if (n > p.L || G < 1 || n % G != 0 || n + G > p.L) return;  // uniform guard
    constexpr int PAD = kLanes + 1;
    const int BD = p.B * p.D;
    const int l = blockIdx.y;
    const int cb = blockIdx.x * kLanes;
    batched_copy(kLanes * G, threadIdx.x, blockDim.x,
        [&](int i) {
            const int k = i % G, ch = cb + i / G;
            return ch < BD ? p.buf[act_row(p, l, ch / p.D, ch % p.D) + n + k] : 0.f;
        },
        [&](int i, float v) { sm[(i % G) * PAD + i / G] = v; });
    __syncthreads();
    // ring += staged sums: load a batch of ring entries, then store the sums
    batched_copy(kLanes * G, threadIdx.x, blockDim.x,
        [&](int i) {
            const int ln = i & (kLanes - 1), k = i / kLanes;
            return cb + ln < BD ? p.ar[ring(p, n + 1 + k, l) + cb + ln] + sm[k * PAD + ln] : 0.f;
        },
        [&](int i, float v) {
            const int ln = i & (kLanes - 1), k = i / kLanes;
            if (cb + ln < BD) p.ar[ring(p, n + 1 + k, l) + cb + ln] = v;
        });
    finish_position(p, n, advance);
}

}  // namespace fi

#include "fi_chunk.h"

namespace fi {

// Tap table of the chunk kernels' helper lanes: per (l, c), 8 runs of 32
// floats, run s holding taps s, s+8, .., s+248 (zero past L, and zero at lags
// 0 and 1, which the red cells add themselves).
__global__ void __launch_bounds__(256) k_taps(Dev p, float *htap) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)p.M * p.D * kChunkTapRow) return;
    const size_t row = i / kChunkTapRow;
    const int e = (int)(i % kChunkTapRow), k = (e / kChunkTaps) + 8 * (e % kChunkTaps);
    htap[i] = k >= 2 && k < p.L ? p.filt[row * (size_t)p.L + k] : 0.f;
}

// Filter heads h^l[c][0..HK-1], channel innermost.
__global__ void __launch_bounds__(256) k_heads(Dev p, float *hh) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)p.M * p.HK * p.D;
    if (i >= total) return;
    const int c = (int)(i % p.D), k = (int)((i / p.D) % p.HK), l = (int)(i / ((size_t)p.D * p.HK));
    hh[i] = k < p.L ? p.filt[filt_row(p, l, c) + k] : 0.f;
}

// ---------------------------------------------------------------------------
// Lazy baseline, sum part: for every (l, b, c), the pending sum at n is the
// whole history term sum_{s=1..n-1} h[n-s] x_s, written into slot n-1; the
// red cells (k_red) then add h[0] x_n.  One workgroup per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_lazy_dot(Dev p, int rd, long long row0) {
    const long long n = position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L) return;
    const long long rowi = row0 + blockIdx.x;
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
        p.ar[ring(p, n, l) + (size_t)b * p.D + c] = tot;
    }
}

// ---------------------------------------------------------------------------
// Eager baseline ([S] "Vergleichsmethoden", Eager: every future contribution
// computed at once): after the red cells of position n have put x_n into the
// history, x_n is pushed into the pending sum of every later position of its
// row, t = n+1 .. L: h[t-n] x_n.  The sum of n+1 is then complete and goes to
// the ring slot the next red cells read; later ones stay in the history row
// (slot t-1, overwritten by x_t when t is reached).  Rows row0 + blockIdx.y,
// 2048 targets per workgroup along x.
// ---------------------------------------------------------------------------
constexpr int kEagerSpan = 2048;
__global__ void __launch_bounds__(256) k_eager_push(Dev p, int rd, long long row0) {
    const long long n = position_of(p, rd);
    if (n >= p.L) return;
    const long long rowi = row0 + blockIdx.y;
    const int b = (int)((rowi / p.D) % p.B), c = (int)(rowi % p.D);
    const int l = (int)(rowi / ((long long)p.D * p.B));
    float *row = p.buf + act_row(p, l, b, c);
    const float *h = p.filt + filt_row(p, l, c);
    const float xn = row[n - 1];
    const long long t0 = n + 1 + (long long)blockIdx.x * kEagerSpan;
    const long long t1 = min(p.L, t0 + kEagerSpan - 1);
    for (long long t = t0 + threadIdx.x; t <= t1; t += blockDim.x) {
        const float v = h[t - n] * xn;
        if (t == n + 1)
            p.ar[ring(p, n + 1, l) + (size_t)b * p.D + c] = row[n] + v;
        else
            row[t - 1] += v;
    }
}

// ---------------------------------------------------------------------------
// Eager prefill ([R] prefill is eager, so the prompt's activations can be
// dropped; [S] "Einschraenkungen": prefill dominates long prompts).  The state
// it leaves is that of P teacher-forced positions: every gray block after
// n <= P done, so later positions run the same schedule.  Per layer l, with all
// of the layer's prompt inputs in the history:
//   k_pre_near  pairs inside one aligned block of G positions (the gray blocks
//               below G): pre[(b,c)][t-1] = sum h[t-s] x_s, t <= P;
//   k_pre_fft   the FFT blocks of edge >= G (fi_fft_kernels.h), adding to pre;
//   k_pre_red   the red cells of every t <= P, then the next layer's inputs.
// 1-D grids over (b, c) x positions; P is a multiple of G.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_pre_in(Dev p, const float *x, long long P) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const long long BD = (long long)p.B * p.D;
    if (i >= (size_t)(BD * P)) return;
    const long long k = (long long)(i / P), t = (long long)(i % P);
    p.buf[(size_t)k * p.L + t] = x[(size_t)t * BD + k];   // layer 0 rows come first
}

// One workgroup per (b, c) and aligned block of G <= 256 positions: the
// block's inputs and taps 0..G-1 staged in LDS, one target per thread.
constexpr int kPreNearMax = 256;
__global__ void __launch_bounds__(kPreNearMax) k_pre_near(Dev p, int l, long long P, int G, float *pre,
                                                          int pstride) {
    __shared__ float xs[kPreNearMax], hs[kPreNearMax];
    const long long nblk = P / G;
    const long long k = blockIdx.x / nblk;                   // (b, c) of layer l
    const long long s0 = (blockIdx.x % nblk) * G;            // the block's first slot
    const int c = (int)(k % p.D), i = threadIdx.x;
    const float *x = p.buf + ((size_t)l * p.B * p.D + k) * (size_t)p.L + s0;
    if (i < G) {
        xs[i] = x[i];
        hs[i] = p.filt[filt_row(p, l, c) + i];
    }
    __syncthreads();
    if (i >= G) return;
    float acc = 0.f;                                         // target slot s0 + i: inputs s0 .. s0+i-1
    for (int j = 0; j < i; ++j) acc = fmaf(hs[i - j], xs[j], acc);
    pre[(size_t)k * pstride + s0 + i] = acc;
}

__global__ void __launch_bounds__(256) k_pre_red(Dev p, int l, long long P, const float *pre, int pstride,
                                                 float *yout) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const long long BD = (long long)p.B * p.D;
    if (i >= (size_t)(BD * P)) return;
    const long long k = (long long)(i / P), t = (long long)(i % P) + 1;
    const int c = (int)(k % p.D);
    const float x = p.buf[((size_t)l * BD + k) * p.L + t - 1];
    const float y = fmaf(p.filt[filt_row(p, l, c)], x, pre[(size_t)k * pstride + t - 1]);
    if (p.recx) {
        const size_t r = ((size_t)(t - 1) * p.M + l) * BD + k;
        p.recx[r] = x;
        p.recy[r] = y;
    }
    if (l + 1 < p.M) {
        p.buf[((size_t)(l + 1) * BD + k) * p.L + t - 1] = apply_map(p.map, y);
    } else {
        p.ylast[(size_t)(t - 1) * BD + k] = y;
        if (yout) yout[(size_t)(t - 1) * BD + k] = y;
        if (t == P) p.xin[(size_t)((P + 1) & 1) * BD + k] = apply_map(p.fb, y);
    }
}

// ---------------------------------------------------------------------------
// External-block mode: the red cell of one layer at position n for all (b, c):
// y = pending + h0 * q, and q becomes the layer input at n.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_red_layer(Dev p, int rd, int l, const float *q, float *y) {
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int BD = p.B * p.D;
    const int chain = blockIdx.x * blockDim.x + threadIdx.x;
    if (chain < BD) {
        const int c = chain % p.D;
        const float x = q[chain];
        const float v = fmaf(p.hh[head(p, l, 0, c)], x, p.ar[ring(p, n, l) + chain]);
        p.xr[ring(p, n, l) + chain] = x;
        if (p.recx) {
            const size_t r = ((size_t)(n - 1) * p.M + l) * BD + chain;
            p.recx[r] = x;
            p.recy[r] = v;
        }
        y[chain] = v;
        if (l == p.M - 1) p.ylast[(size_t)(n - 1) * BD + chain] = v;
    }
}

}  // namespace fi
