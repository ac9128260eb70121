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

constexpr int kLanes = 64;  // chains per block: one per lane, so every access is coalesced
// Threads of a direct-block workgroup (one wave runs the red cells, the rest
// stage rows from memory: the staging is the critical path from U = 2 on, and
// sixteen waves measured 25-50% faster than four there) and of the
// ring <-> history copies at FFT positions.
constexpr int kDirectThreads = 1024;
constexpr int kRingThreads = 1024;
constexpr int kChunkThreads = 1024;  // chunk workgroups: wave 0 + up to 15 helper waves

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

// ---------------------------------------------------------------------------
// All positions of one chunk (cb, cb + G] (cb a multiple of G, the edge of
// the first FFT class, G <= 256) for maps that act channel by channel.  Then
// every (b, c) chain is independent through all layers, and so is every gray
// block below G: their sources and targets lie in the same chunk (a block
// after n has U = lowbit(n) < G, so n + U never passes the next multiple of
// G).  One workgroup owns CH chains and all M layers and runs the chunk's G
// positions back to back, with a barrier between positions and no launch.
//
// The gray blocks of edge U < G inside a chunk cover every pair s < t of the
// chunk exactly once, so their sum into target t is the causal dot product
// over the chunk.  It is formed here target by target:
//   pend(t) = fft(t) + sum_{k=2..} h[k] x_{t-k}  (helpers, during position t-1)
//           + h[1] x_{t-1}                       (chain lane, at position t)
// so only the last term waits for the position before.  One LDS slot per
// (position, row) holds the FFT pending sum (loaded from the row-major
// history), then the finished sum, then the input x_t (the pages' activation
// reuse); at the end the slots are the inputs the next FFT block reads.
//
// Waves (16): wave 0 runs the red cells, one chain per lane; the other waves
// of its SIMD (4, 8, 12: waves go to the four SIMDs in turn) stay off the
// arithmetic, and wave 4 stamps each position once its barrier has passed;
// the twelve remaining waves are helpers, eight lanes per row.
//
// LDS: heads h01[R] (h[0], h[1]); slots xp[G][kChunkSlot], slot s at row
// G-1-s (reversed, so that the taps of a helper lie at increasing addresses:
// immediate offsets, read in pairs); a zero row G; teacher-forced inputs
// xs[G][CH].  Rows rho = j * M + l for chain c0 + j, layer l.
//
// Global memory inside the position loop: the chain's last-layer output, the
// helpers' history stores (one 128-byte line per row every 32 positions, for
// the FFT block at the chunk's end) and wave 4's stamps.
// ---------------------------------------------------------------------------
constexpr int kChunkTaps = 32;       // taps per helper lane: h[seg + 8m], m < 32 (G <= 256)
constexpr int kChunkTapRow = 8 * kChunkTaps;   // tap-table floats per (l, c): taps 0..255
constexpr int kChunkRegLayers = 20;  // stacks up to this depth keep a chain's layers in registers
constexpr int kChunkHelperWaves = 12;
constexpr int kChunkMaxRows = kChunkHelperWaves * kLanes / 8;   // 96
// floats per slot: >= the rows, and 8 slots apart = 15 x 256 bytes (one
// read2st64 reaches two taps); the eight lanes of a row then hit distinct banks
constexpr int kChunkSlot = 120;
// zero row after the slots: a helper tap that lies before the chunk reads it
constexpr int kChunkZeroRows = 1;
// chunk kernel variants: records every layer's input and output; both maps tanh
constexpr int kChunkRec = 1, kChunkTanh = 2;
// 0: the chain reads a position's pending sums when it starts (one barrier per
// position); q > 0: a second barrier after layer q M / 4, where the chain
// reads the next position's sums while its remaining layers run
constexpr int kChunkMidQ = 0; 

// Red cells of the chunk's positions for one chain per lane of wave 0, all
// layers; one barrier per position, as in the other waves.  MT = M layers:
// heads and the previous position's inputs in registers, the pending sums of
// the position read from LDS in one batch, then straight-line code with no
// branch between layers.  Lanes without a chain run the same code on chain
// 0's data and store nothing.  MT = 0: any depth, one layer at a time from LDS.
template <int MT, bool REC, bool TANH_ALL>
__device__ __forceinline__ void chain_run(const Dev &p, float *xp, int G, const float2 *hz, long long cb, int j,
                                          int chain, bool on, const float *xs, int CH) {
    const int BD = p.B * p.D, M = p.M;
    const int jr = on ? j : 0;                 // the chain whose LDS data this lane reads
    constexpr int NR = MT > 0 ? MT : 1;
    constexpr int MID = kChunkMidQ > 0 && MT > 0 ? MT * kChunkMidQ / 4 : -1;
    float h0[NR], h1[NR], xq[NR], pn[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const float2 v = MT > 0 ? hz[jr * M + k] : make_float2(0.f, 0.f);
        h0[k] = v.x;
        h1[k] = v.y;
        xq[k] = 0.f;                           // slot -1: its tap-1 term is in the FFT sums
        pn[k] = MID >= 0 ? xp[(size_t)(G - 1) * kChunkSlot + jr * M + k] : 0.f;   // slot 0
    }
    float xf = on ? p.xin[(size_t)((cb + 1) & 1) * BD + chain] : 0.f;   // feedback input
    const bool map_id = !TANH_ALL && p.map != 0, fb_id = !TANH_ALL && p.fb != 0;
    for (int i = 0; i < G; ++i) {
        const long long t = cb + 1 + i;        // position
        float x = xs ? xs[i * CH + jr] : xf;   // teacher-forced inputs, staged in LDS
        float *cur = xp + (size_t)(G - 1 - i) * kChunkSlot + jr * M;   // this chain's layers at slot i
        float y = 0.f;
        if constexpr (MT > 0) {
            float a[MT];
#pragma unroll
            for (int k = 0; k < MT; ++k) a[k] = fmaf(h1[k], xq[k], MID >= 0 ? pn[k] : cur[k]);   // + tap 1 of slot i-1
#pragma unroll
            for (int k = 0; k < MT; ++k) {
                if (k == MID) {
                    __syncthreads();           // the helper sums of slot i+1 are complete
                    if (i + 1 < G) {
#pragma unroll
                        for (int kk = 0; kk < MT; ++kk) pn[kk] = cur[kk - kChunkSlot];   // slot i+1
                    }
                }
                y = fmaf(h0[k], x, a[k]);
                xq[k] = x;
                if constexpr (REC) {
                    if (on) {
                        const size_t r = ((size_t)(t - 1) * MT + k) * BD + chain;
                        p.recx[r] = x;
                        p.recy[r] = y;
                    }
                }
                const float th = tanh_chain(y);
                if constexpr (TANH_ALL) {
                    x = th;
                } else {
                    x = (k + 1 < MT ? map_id : fb_id) ? y : th;   // both maps evaluated, one selected
                }
            }
            if (on) {
#pragma unroll
                for (int k = 0; k < MT; ++k) cur[k] = xq[k];
            }
        } else {
            for (int l = 0; l < M; ++l) {
                const float2 h = hz[jr * M + l];
                const float pend = i > 0 ? fmaf(h.y, cur[l + kChunkSlot], cur[l]) : cur[l];
                y = fmaf(h.x, x, pend);
                if (on) cur[l] = x;
                if (REC && on) {
                    const size_t r = ((size_t)(t - 1) * M + l) * BD + chain;
                    p.recx[r] = x;
                    p.recy[r] = y;
                }
                x = apply_map(l + 1 < M ? p.map : p.fb, y);
            }
            if (kChunkMidQ > 0) __syncthreads();
        }
        if (on) p.ylast[(size_t)(t - 1) * BD + chain] = y;
        xf = x;
        __syncthreads();
    }
    if (on) p.xin[(size_t)((cb + G + 1) & 1) * BD + chain] = xf;
}

// Sum over each aligned group of eight lanes, in every lane of the group:
// swaps within quads (lane ^ 1, lane ^ 2), then the mirror within the group.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum8(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);   // row_half_mirror
    return v;
}

template <int NF>
__device__ __forceinline__ float helper_sum(const float *xp, const float *hreg, int row0, int hrho, int G) {
    constexpr int S = 8, SP = kChunkSlot;
    constexpr int NT = NF < 4 ? 8 * (NF + 1) : 32;
    float v[NT];
    const float *base = xp + (size_t)row0 * SP + hrho;
#pragma unroll
    for (int m = 0; m < 8 * NF && m < NT; ++m) v[m] = base[(size_t)m * S * SP];
#pragma unroll
    for (int m = 8 * NF; m < NT; ++m) v[m] = xp[(size_t)min(row0 + S * m, G) * SP + hrho];
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m & 3] = fmaf(hreg[m], v[m], acc[m & 3]);
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <int MT, int MODE>
__global__ void __launch_bounds__(kChunkThreads) k_chunk(Dev p, long long cb, int G, int CH, const float *xseq) {
    constexpr int S = 8;                       // helper lanes per row
    constexpr int SP = kChunkSlot;
    extern __shared__ float sm[];
    const int M = p.M, BD = p.B * p.D, R = CH * M;
    float2 *h01 = (float2 *)sm;                            // [R]
    float *xp = sm + 2 * R;                                // [G][SP], slot s at row G-1-s
    float *xz = xp + (size_t)G * SP;                       // [kChunkZeroRows][SP] zeros: row G
    float *xs = xz + kChunkZeroRows * SP;                  // [G][CH] teacher-forced inputs
    const int c0 = blockIdx.x * CH;
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x / kLanes;
    const int logG = 31 - __clz(G);
    auto grow = [&](int rho) {                             // history row of local row rho
        return ((size_t)(rho % M) * BD + c0 + rho / M) * (size_t)p.L;
    };
    auto frow = [&](int rho) {                             // filter row
        return ((size_t)(rho % M) * p.D + (c0 + rho / M) % p.D) * (size_t)p.L;
    };
    auto trow = [&](int rho) {                             // tap-table row
        return (size_t)(rho % M) * p.D + (c0 + rho / M) % p.D;
    };
    auto live = [&](int rho) { return c0 + rho / M < BD; };

    // helper lanes: row hrho, taps h[seg + 8m] (zero for k < 2: the chain
    // adds tap 1, tap 0 is the red cell's own term); loads issued first
    const int hw = (wave & 3) ? wave - 1 - wave / 4 : -1;
    const int hid = hw * kLanes + lane;
    const int hrho = hid / S, seg = hid & (S - 1);
    const bool helper = hw >= 0 && hrho < R && live(hrho);
    float hreg[kChunkTaps];
    {
        // the lane's 32 taps lie together in the tap table: eight 16-byte loads
        const float4 *tp = (const float4 *)(p.htap + (size_t)(helper ? trow(hrho) : 0) * kChunkTapRow +
                                            seg * kChunkTaps);
#pragma unroll
        for (int q = 0; q < kChunkTaps / 4; ++q) {
            const float4 v = tp[q];
            hreg[4 * q] = v.x;
            hreg[4 * q + 1] = v.y;
            hreg[4 * q + 2] = v.z;
            hreg[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int m = 0; m < kChunkTaps; ++m) {
            const int k = seg + S * m;
            if (!(helper && k >= 2 && k < G)) hreg[m] = 0.f;
        }
    }

    // pending sums of the chunk's positions (rows of the history, G slots
    // each: coalesced reads), the heads, the teacher-forced inputs
    if (G >= 4) {
        const int g4 = logG - 2;                           // float4 per row: G / 4
        for (int e = threadIdx.x; e < (R * G) >> 2; e += blockDim.x) {
            const int rho = e >> g4, s0 = (e & ((G >> 2) - 1)) * 4;
            const float4 v = live(rho) ? *(const float4 *)(p.buf + grow(rho) + cb + s0)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
            float *d = xp + (size_t)(G - 1 - s0) * SP + rho;
            d[0] = v.x;
            d[-SP] = v.y;
            d[-2 * SP] = v.z;
            d[-3 * SP] = v.w;
        }
    } else {
        for (int e = threadIdx.x; e < R * G; e += blockDim.x) {
            const int rho = e >> logG;
            xp[(size_t)(G - 1 - (e & (G - 1))) * SP + rho] = live(rho) ? p.buf[grow(rho) + cb + (e & (G - 1))] : 0.f;
        }
    }
    for (int e = threadIdx.x; e < kChunkZeroRows * SP; e += blockDim.x) xz[e] = 0.f;
    for (int rho = threadIdx.x; rho < R; rho += blockDim.x)
        h01[rho] = live(rho) ? make_float2(p.filt[frow(rho)], p.L > 1 ? p.filt[frow(rho) + 1] : 0.f)
                             : make_float2(0.f, 0.f);
    if (xseq)
        for (int e = threadIdx.x; e < G * CH; e += blockDim.x) {
            const int i = e / CH, j = e % CH;
            xs[e] = c0 + j < BD ? xseq[(size_t)i * BD + c0 + j] : 0.f;
        }
    __syncthreads();

    float *hist = p.buf + (helper ? grow(hrho) + cb : 0);   // a helper row's positions of the chunk
    if (wave == 0) {
        // ---- red cells; the helpers do not share this wave's SIMD
        __builtin_amdgcn_s_setprio(3);
        chain_run<MT, (MODE & kChunkRec) != 0, (MODE & kChunkTanh) != 0>(
            p, xp, G, h01, cb, lane, c0 + lane, lane < CH && c0 + lane < BD, xseq ? xs : nullptr, CH);
    } else if (hw < 0) {
        // ---- waves 4, 8, 12: barriers only; wave 4 stamps each position's end
        for (int i = 0; i < G; ++i) {
            if (kChunkMidQ > 0) __syncthreads();
            __syncthreads();
            if (wave == 4 && lane == 0)
                atomicMax((unsigned long long *)&p.stamps[cb + 1 + i], (unsigned long long)wall_clock64());
        }
    } else {
        // ---- helpers: during position i, the pending sum of slot i+1 but for
        // its tap-1 term: fft + sum_{k>=2} h[k] x_{i+1-k}.  Tap m of a lane
        // (k = seg + 8m) reads slot i+1-k at row row0 + 8m.  Taps come in four
        // groups of eight m; the first nf = (i+2)/64 groups exist in every
        // lane, the next one in some (its other lanes read the zero rows past
        // the chunk's first slot), the rest in none.  nf is uniform and picks
        // a branch-free body, so all of a position's reads are in flight.
        for (int i = 0; i < G; ++i) {
            // every 32 positions, the inputs of the last 32 into the history,
            // for the FFT block at the chunk's end: one whole 128-byte line per
            // row, 16 bytes per lane (slots i-32+4seg .. +3, from row G-i+31-4seg down)
            if (helper && i >= 32 && (i & 31) == 0) {
                const float *src = xp + (size_t)(G - i + 31 - 4 * seg) * SP + hrho;
                *(float4 *)(hist + i - 32 + 4 * seg) = make_float4(src[0], src[-SP], src[-2 * SP], src[-3 * SP]);
            }
            if (i + 1 < G) {
                const int row0 = G - 2 - i + seg;
                float acc;
                switch ((i + 2) >> 6) {
                    case 0: acc = helper_sum<0>(xp, hreg, row0, hrho, G); break;
                    case 1: acc = helper_sum<1>(xp, hreg, row0, hrho, G); break;
                    case 2: acc = helper_sum<2>(xp, hreg, row0, hrho, G); break;
                    case 3: acc = helper_sum<3>(xp, hreg, row0, hrho, G); break;
                    default: acc = helper_sum<4>(xp, hreg, row0, hrho, G); break;
                }
                acc = sum8(acc);
                if (helper && seg == 0) xp[(size_t)(G - 2 - i) * SP + hrho] += acc;
            }
            if (kChunkMidQ > 0) __syncthreads();   // the chain reads slot i+1
            __syncthreads();                   // the chain has written slot i
        }
    }

    // the remaining inputs into the history: the last 32 slots as above, or
    // all of a chunk shorter than 32
    if (helper) {
        if (G >= 32) {
            const float *src = xp + (size_t)(31 - 4 * seg) * SP + hrho;   // slot G-32+4seg at row 31-4seg
            *(float4 *)(hist + G - 32 + 4 * seg) = make_float4(src[0], src[-SP], src[-2 * SP], src[-3 * SP]);
        } else {
            for (int sl = seg; sl < G; sl += S) hist[sl] = xp[(size_t)(G - 1 - sl) * SP + hrho];
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const long long n = cb + G;           // published: the FFT block of n reads slot (n-1)&1
        p.st->pos[(n - 1) & 1] = n - 1;
        p.st->pos[n & 1] = n;
    }
}

// End of an FFT position reached from a chunk: n is published and stamped
// once every gray-block kernel of n has finished (one thread).
__global__ void __launch_bounds__(64) k_publish(Dev p, long long n) {
    if (threadIdx.x == 0) {
        p.stamps[n] = (long long)wall_clock64();
        p.st->pos[(n - 1) & 1] = n - 1;
        p.st->pos[n & 1] = n;
    }
}

// Tap table of the chunk kernels' helper lanes: per (l, c), 8 runs of 32
// floats, run s holding taps s, s+8, .., s+248 (zero past L).
__global__ void __launch_bounds__(256) k_taps(Dev p, float *htap) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)p.M * p.D * kChunkTapRow) return;
    const size_t row = i / kChunkTapRow;
    const int e = (int)(i % kChunkTapRow), k = (e / kChunkTaps) + 8 * (e % kChunkTaps);
    htap[i] = k < p.L ? p.filt[row * (size_t)p.L + k] : 0.f;
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
// Gray blocks of all layers by FFT, U = 2^LOGN (complex transform of U points
// carries the 2U-point real circular convolution).  One team of TT threads per
// (l, b, c) block; the red cells at n have already run.
//   spec: per (l, c), U/2 float4 in pair order (see k_spectrum), scaled by 1/U.
// ---------------------------------------------------------------------------
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
#pragma unroll
    for (int m = 0; m < HALF0; ++m) {
        v[m] = active ? xsrc[lt + (m << QLOG0)] : make_float2(0.f, 0.f);
        v[m + HALF0] = make_float2(0.f, 0.f);
    }
    dif_group<R0, true>(v, lt, LOGN, p.twid, p.logNT);
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGN, 1>(X, lt, p.twid, p.logNT);
    // this thread's spectrum pairs, loaded only now: held across the forward
    // transform they would cost the registers of a fourth wave per SIMD
    constexpr int PAIRS = (N / 2 + TT - 1) / TT;
    float4 gs[PAIRS];
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        gs[m] = (active && e < N / 2) ? sp[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    // bins of the real transform times the filter spectrum, re-packed for the inverse
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
        const int e = lt + m * TT;
        if (e >= N / 2) break;
        const float4 g = gs[m];
        if (e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            const float Z0 = (C0.x + C0.y) * g.x;
            const float ZN = (C0.x - C0.y) * g.y;
            X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
            X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w));
        } else {
            const PairSlot ps = pair_slot(LOGN, e);
            const int p1 = lpad(ps.pj), p2 = lpad(ps.pm);
            const float2 W = p.ptw[N / 2 + e];
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
    if (active) {  // the accumulators, like the spectrum, are read late
        float2 acc[HALF0];
#pragma unroll
        for (int m = 0; m < HALF0; ++m) acc[m] = adst[lt + (m << QLOG0)];
#pragma unroll
        for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    }
    finish_position(p, n, advance);
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
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
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
    for (int m = 0; m < 16; ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGM, 1>(X, lt, p.twid, p.logNT);
}

// Inverse transform of one half from X (items already re-packed; the caller
// has synchronised) and its accumulation into dst[0..M): the odd half
// subtracts W_{2M}^{-m} v, the even half adds v.
template <int LOGM, bool ODD>
__device__ __forceinline__ void half_inverse_acc(const Dev &p, float2 *X, int lt, bool active, float2 *dst) {
    using S = FftShape<LOGM>;
    constexpr int R0 = S::R0, QLOG0 = S::QLOG0;
    inverse_groups<LOGM, S::NPASS - 1>(X, lt, p.twid, p.logNT);
    float2 v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = X[lpad(lt + (m << QLOG0))];
    dit_group<R0>(v, lt, LOGM, p.twid, p.logNT);
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
            const PairSlot ps = half_slot<LOGM, ODD>(e);
            const int p1 = lpad(ps.pj), p2 = lpad(ps.pm);
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
    for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    forward_groups<LOGV, 1>(X, lt, p.twid, p.logNT);
    __syncthreads();
    float4 *dst = scratch + ((size_t)tile * K + i) * (N / 2);
    for (int e = lt; e < N / 2; e += TT) {
        if (e == 0) {
            const float2 C0 = X[0];
            const float2 Ch = X[lpad(1)];
            dst[0] = make_float4(C0.x + C0.y, C0.x - C0.y, Ch.x, -Ch.y);
        } else {
            const PairSlot ps = pair_slot(LOGV, e);
            float2 A1, A2;
            real_bins(X[lpad(ps.pj)], X[lpad(ps.pm)], p.ptw[N / 2 + e], A1, A2);
            dst[e] = make_float4(A1.x, A1.y, A2.x, A2.y);
        }
    }
}

// k_fft_sub_inv: per (l, b, c, o), Z = sum_i A_i * G_{K+o-i}, then the inverse
// transform and accumulation of its exact upper half into output sub-block o.
// One launch covers output sub-blocks o0 .. o0+nO-1.  nfix > 0 names the
// position directly (a launch that runs after later positions have already
// overwritten the position slots).
template <int LOGV>
__global__ void __launch_bounds__(FftShape<LOGV>::TPB) k_fft_sub_inv(Dev p, int rd, const float4 *__restrict__ scratch,
                                                                     const float4 *__restrict__ spec, int K,
                                                                     int o0, int nO, long long nfix, int advance) {
    using S = FftShape<LOGV>;
    constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
    __shared__ float2 smem[S::LDS];
    const int lt = threadIdx.x;
    const long long U = (long long)K * N;
    const long long n = nfix > 0 ? nfix : position_of(p, rd);
    const long long t = n - 1;
    if (n > p.L || n % U != 0 || n + U > p.L) return;  // uniform guard
    long long tile;
    int o;
    xcd_tile(blockIdx.x, (long long)p.M * p.B * p.D, nO, tile, o);
    o += o0;
    const int c = (int)(tile % p.D);
    const int l = (int)(tile / ((long long)p.D * p.B));
    const size_t row = (size_t)tile * (size_t)p.L;
    float2 *adst = reinterpret_cast<float2 *>(p.buf + row + t + 1 + (long long)o * N);
    const float4 *A = scratch + (size_t)tile * K * (N / 2);
    const float4 *G = spec + ((size_t)l * p.D + c) * (size_t)(2 * K - 1) * (N / 2);
    float2 *X = smem;
    // Z = sum_i A_i * G_{K+o-i} for this thread's pairs, four pairs at a time.
    // Step s covers chunk s / K and sub-block i = s % K; the loads of step
    // s + 1 are in flight while step s multiplies (K is even).
    constexpr int PAIRS = (N / 2 + TT - 1) / TT;
    constexpr int CH = 4;
    static_assert(PAIRS % CH == 0, "pairs per thread");
    const int steps = (PAIRS / CH) * K;
    auto load = [&](int st, float4(&a)[CH], float4(&g)[CH]) {
        const int m0 = (st / K) * CH, i = st % K;
        const float4 *Ai = A + (size_t)i * (N / 2);
        const float4 *Gi = G + (size_t)(K + o - i - 1) * (N / 2);
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            const int j = lt + (m0 + m) * TT;
            a[m] = Ai[j];
            g[m] = Gi[j];
        }
    };
    float4 Z[CH];
    auto mac = [&](int st, const float4(&a)[CH], const float4(&g)[CH]) {
        const int m0 = (st / K) * CH;
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            if (lt + (m0 + m) * TT == 0) {  // (G_0, G_N) real, G_{N/2} complex
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
    // re-pack the finished chunk for the inverse transform
    auto flush = [&](int m0) {
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            const int j = lt + (m0 + m) * TT;
            if (j == 0) {
                const float Z0 = Z[m].x, ZN = Z[m].y;
                X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN));
                X[lpad(1)] = make_float2(Z[m].z, -Z[m].w);
            } else {
                const PairSlot ps = pair_slot(LOGV, j);
                float2 D1, D2;
                pack_inverse(make_float2(Z[m].x, Z[m].y), make_float2(Z[m].z, Z[m].w), p.ptw[N / 2 + j], D1, D2);
                X[lpad(ps.pj)] = D1;
                X[lpad(ps.pm)] = D2;
            }
            Z[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
#pragma unroll
    for (int m = 0; m < CH; ++m) Z[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 a0[CH], g0[CH], a1[CH], g1[CH];
    load(0, a0, g0);
    for (int st = 0; st < steps; st += 2) {
        load(st + 1, a1, g1);
        mac(st, a0, g0);
        if (st + 2 < steps) load(st + 2, a0, g0);
        mac(st + 1, a1, g1);
        if ((st + 1) % K == K - 1) flush(((st + 1) / K) * CH);
    }
    __syncthreads();
    inverse_groups<LOGV, S::NPASS - 1>(X, lt, p.twid, p.logNT);
    float2 v[1 << R0];
#pragma unroll
    for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
    dit_group<R0>(v, lt, LOGV, p.twid, p.logNT);
    float2 acc[HALF0];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) acc[m] = adst[lt + (m << QLOG0)];
#pragma unroll
    for (int m = 0; m < HALF0; ++m) adst[lt + (m << QLOG0)] = cadd(acc[m], v[m + HALF0]);
    finish_position(p, n, advance);
}

// ---------------------------------------------------------------------------
// Lazy baseline, sum part: for every (l, b, c), the pending sum at n is the
// whole history term sum_{s=1..n-1} h[n-s] x_s, written into slot n-1; the
// red cells (k_red) then add h[0] x_n.  One workgroup per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_lazy_dot(Dev p, int rd) {
    const long long n = position_of(p, rd);
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
        p.ar[ring(p, n, l) + (size_t)b * p.D + c] = tot;
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
