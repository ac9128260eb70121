// The chunk kernel: all positions between two FFT positions as one launch
// for maps that act channel by channel (see the comment on k_chunk).
//
// Flash Inference (arXiv 2410.12982), summary page, "Kachelung-Strategie
// (Algorithmus 1)": the gray blocks of edge below G inside a chunk cover every
// pair s < t of the chunk exactly once; "LCSM-Inferenz-Algorithmus"
// (Algorithm 2): the red cells of a position run layer after layer.
#pragma once
#include <type_traits>

#include "fi_device.h"
#include "fi_tanh.h"

namespace fi {

constexpr int kChunkThreads = 1024;  // chunk workgroups: wave 0 + up to 15 helper waves

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
// immediate offsets); zero rows G .. G+63; teacher-forced
// inputs xs[G][CH].  Rows rho = j * M + l for chain c0 + j, layer l.
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
static_assert(kChunkMaxRows <= kChunkThreads - kLanes, "one head row per set-up thread");
// Floats per slot: >= the rows, and 8 mod 32.  A multiple of 8 lets one
// read2st64 fetch two taps of a lane (taps 8 slots apart: 13 x 256 bytes);
// 8 mod 32 puts the four lanes of a row that share a half-wave (slots seg
// apart, seg = 0..3 or 4..7) on four banks 8 apart, which the eight rows of
// the half-wave fill without a conflict (see the helper lanes in k_chunk).
constexpr int kChunkSlot = 104;
static_assert(kChunkSlot >= kChunkMaxRows && kChunkSlot % 32 == 8, "slot width");
// zero rows after the slots: the helper taps that lie before the chunk read them
constexpr int kChunkZeroRows = 64;
// positions a chain stays on a costlier tanh pass after the cheaper one failed
constexpr int kChainFullRun = 128;
// chunk kernel variants: records every layer's input and output; both maps tanh
constexpr int kChunkRec = 1, kChunkTanh = 2;

// Red cells of the chunk's positions for one chain per lane of wave 0, all
// layers; one barrier per position, as in the other waves.  MT = M layers:
// heads and the previous position's inputs in registers, the pending sums of
// the position read from LDS in one batch, then straight-line code with no
// branch between layers.  Lanes without a chain run the same code on chain
// 0's data, feedback input included (so their values, and the range vote,
// are chain 0's), and store nothing.  MT = 0: any depth, one layer at a time
// from LDS.
template <int MT, bool REC, bool TANH_ALL>
__device__ __forceinline__ void chain_run(const Dev &p, float *xp, int G, const float2 *hz, long long cb, int j,
                                          int chain, bool on, const float *xs, int CH, float xf) {
    const int BD = p.B * p.D, M = p.M;
    const int jr = on ? j : 0;                 // the chain whose LDS data this lane reads
    constexpr int NR = MT > 0 ? MT : 1;
    float h0[NR], h1[NR], xq[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const float2 v = MT > 0 ? hz[jr * M + k] : make_float2(0.f, 0.f);
        h0[k] = v.x;
        h1[k] = v.y;
        xq[k] = 0.f;                           // slot -1: its tap-1 term is in the FFT sums
    }
    const bool map_id = !TANH_ALL && p.map != 0, fb_id = !TANH_ALL && p.fb != 0;
    int full_left = 0;                         // wave-uniform: positions left on the full tanh
    int small_left = 0;                        // and on the polynomial pieces
    for (int i = 0; i < G; ++i) {
        const long long t = cb + 1 + i;        // position
        float x = xs ? xs[i * CH + jr] : xf;   // teacher-forced inputs, staged in LDS
        float *cur = xp + (size_t)(G - 1 - i) * kChunkSlot + jr * M;   // this chain's layers at slot i
        float y = 0.f;
        if constexpr (MT > 0) {
            float a[MT];
#pragma unroll
            for (int k = 0; k < MT; ++k) a[k] = fmaf(h1[k], xq[k], cur[k]);   // + tap 1 of slot i-1
            const float x0 = x;
            // largest y^2 of a polynomial pass: every |y| < 0.72 exactly when
            // every rounded y^2 < kTanhSmallSq (rounding is monotone, and the
            // rounded square of 0.72f's predecessor lies below it), and every
            // |y| < 0.125 exactly when every rounded y^2 < 2^-6; so one vote per
            // position, on squares the polynomials form anyway, decides
            float s2max = 0.f;
            // the position's layers with tanh by piece TIER: 0 the first piece
            // alone (for positions where every |y| stays below 0.125), 1 the
            // polynomial pieces (below 0.72), 2 the full tanh
            auto layers = [&](auto tier) {
                constexpr int TIER = decltype(tier)::value;
                x = x0;
#pragma unroll
                for (int k = 0; k < MT; ++k) {
                    y = fmaf(h0[k], x, a[k]);
                    xq[k] = x;
                    if constexpr (REC) {
                        if (on) {
                            const size_t r = ((size_t)(t - 1) * MT + k) * BD + chain;
                            p.recx[r] = x;
                            p.recy[r] = y;
                        }
                    }
                    const float th = TIER == 2 ? tanh_chain(y) : TIER == 1 ? tanh_small(y) : tanh_tiny(y);
                    if constexpr (TIER < 2) s2max = fmaxf(s2max, y * y);
                    if constexpr (TANH_ALL) {
                        x = th;
                    } else {
                        x = (k + 1 < MT ? map_id : fb_id) ? y : th;   // both maps evaluated, one selected
                    }
                }
            };
            if constexpr (TANH_ALL) {
                // Both maps tanh.  A position runs the cheapest pass first: the
                // first piece alone, which keeps the polynomial's higher terms
                // and the exponential off the chain.  If some lane of the wave
                // left its range, the position runs again with the next pass
                // (same values where both apply), and so do the next
                // kChainFullRun positions before the cheaper pass is tried
                // again (activations that stay large then cost one extra pass
                // per kChainFullRun positions).
                using T0 = std::integral_constant<int, 0>;
                using T1 = std::integral_constant<int, 1>;
                using T2 = std::integral_constant<int, 2>;
                if (full_left == 0) {
                    if (small_left == 0) {
                        s2max = 0.f;
                        layers(T0{});
                        if (__builtin_amdgcn_ballot_w64(!(s2max < kTanhTinySq))) small_left = kChainFullRun + 1;
                    }
                    if (small_left > 0) {
                        s2max = 0.f;
                        layers(T1{});
                        if (__builtin_amdgcn_ballot_w64(!(s2max < kTanhSmallSq))) {
                            // after the full run, the polynomial pass is the one tried again
                            full_left = kChainFullRun + 1;
                            small_left = kChainFullRun + 1;
                        }
                        --small_left;
                    }
                }
                if (full_left > 0) {
                    layers(T2{});
                    --full_left;
                }
            } else {
                layers(std::integral_constant<int, 2>{});
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
        }
        if (on) p.ylast[(size_t)(t - 1) * BD + chain] = y;
        xf = x;
        __syncthreads();
    }
    if (on) p.xin[(size_t)((cb + G + 1) & 1) * BD + chain] = xf;
}

// Sum over the eight lanes of a helper row (lanes 4q..4q+3 and 32+4q..+3 of
// the wave), valid in the row's lanes of the lower half: swaps within quads
// (lane ^ 1, lane ^ 2), then the quad of the upper half (v_permlane32_swap:
// its second result holds lanes 32..63 in lanes 0..31).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum8(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    const auto hi = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return v + __uint_as_float(hi[1]);
}

// Lags of a chunk split between the two kinds of helper work: a lane's taps
// m < kChunkPullTaps (lags k = seg + 8m below 8 kChunkPullTaps) are pulled,
// target by target, one position ahead; taps m >= kChunkPullTaps (the longer
// lags, only in chunks longer than 8 kChunkPullTaps) are pushed from each
// source one position after it is known.
constexpr int kChunkPullTaps = 24;
// s_waitcnt vmcnt(0), the other counters left free (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;
static_assert(kChunkPullTaps % 8 == 0 && kChunkPullTaps <= kChunkTaps, "pulled taps come in groups of eight");

// f(std::integral_constant<int, v>) for the v in [0, N] equal to the runtime
// value (uniform over the wave: a scalar branch to a body with fixed offsets).
template <int N, int V = 0, typename F>
__device__ __forceinline__ void dispatch(int v, F &&f) {
    if constexpr (V < N) {
        if (v == V) {
            f(std::integral_constant<int, V>{});
            return;
        }
        dispatch<N, V + 1>(v, f);
    } else {
        f(std::integral_constant<int, N>{});
    }
}

// A helper lane's partial sum over its taps m < 8 (NF + 1) (tap m: slot row
// row0 + 8m, register hreg[m]).  Taps of group NF that lie before the chunk's
// first slot read the zero rows after the slots (rows G .. G+63: with
// NF = min((i+2)/64, kChunkPullTaps/8 - 1), row0 + 8m never passes G+63), so
// every tap is a plain read at a fixed offset.
template <int NF>
__device__ __forceinline__ float helper_sum(const float *xp, const float *hreg, int row0, int hrho, bool lag01) {
    constexpr int S = 8, SP = kChunkSlot;
    constexpr int NT = 8 * (NF + 1);
    static_assert(NT <= kChunkPullTaps, "pulled taps");
    float v[NT];
    const float *base = xp + (size_t)row0 * SP + hrho;
#pragma unroll
    for (int m = 0; m < NT; ++m) v[m] = base[(size_t)m * S * SP];
    // lags 0 and 1 (tap 0 of lanes 0 and 1) are the slots of the target and
    // of the position being computed, whose values are not settled: their
    // zero taps must not meet an infinity there
    if (lag01) v[0] = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m & 3] = fmaf(hreg[m], v[m], acc[m & 3]);
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// A helper lane's push of the source x (slot i-1, known from position i on)
// into the pending sums of its targets t = i-1 + seg + 8m for its pushed taps
// m = kChunkPullTaps .. kChunkPullTaps+C-1, which lie inside the chunk in every
// lane (target of tap m at row rowp - 8 (m - kChunkPullTaps)), and for tap
// m = kChunkPullTaps+C where its row is still a slot (row >= 0: this lane's
// target inside the chunk).  C is uniform over the wave, so the reads and
// writes are plain accesses at fixed offsets.  Each target belongs to one
// lane of its row (its lag fixes seg and m), so no two lanes update one sum.
template <int C>
__device__ __forceinline__ void helper_push(float *xp, const float *hreg, int rowp, int hrho, float x) {
    constexpr int S = 8, SP = kChunkSlot, P = kChunkPullTaps;
    if constexpr (C > 0) {
        // from the lowest row up, so that every access is the base plus a
        // non-negative immediate
        float *b = xp + (size_t)(rowp - S * (C - 1)) * SP + hrho;
        float v[C];
#pragma unroll
        for (int c = 0; c < C; ++c) v[c] = b[(size_t)(C - 1 - c) * S * SP];
#pragma unroll
        for (int c = 0; c < C; ++c) b[(size_t)(C - 1 - c) * S * SP] = fmaf(hreg[P + c], x, v[c]);
    }
    if constexpr (P + C < kChunkTaps) {
        const int r = rowp - S * C;
        if (r >= 0) {
            float *d = xp + (size_t)r * SP + hrho;
            *d = fmaf(hreg[P + C], x, *d);
        }
    }
}

template <int MT, int MODE>
__global__ void __launch_bounds__(kChunkThreads) k_chunk(Dev p, long long cb_arg, int G, int CH, const float *xseq) {
    // cb < 0: the chunk follows the position published in the state (graph
    // replays); a chunk starts after a multiple of G, so that position is even
    // and sits in slot 0
    const long long cb = cb_arg >= 0 ? cb_arg : p.st->pos[0];
    constexpr int S = 8;                       // helper lanes per row
    constexpr int SP = kChunkSlot;
    extern __shared__ float sm[];
    const int M = p.M, BD = p.B * p.D, R = CH * M;
    float2 *h01 = (float2 *)sm;                            // [R]
    float *xp = sm + 2 * R;                                // [G][SP], slot s at row G-1-s
    float *xz = xp + (size_t)G * SP;                       // [kChunkZeroRows][SP] zeros: rows G..
    float *xs = xz + kChunkZeroRows * SP;                  // [G][CH] teacher-forced inputs
    const int c0 = blockIdx.x * CH;
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x / kLanes;
    // the chain's feedback input, loaded first.  The first touch of its page
    // after the FFT blocks can take several microseconds: wave 0 loads nothing
    // else before the position loop, and the other waves' set-up below hides it
    const int jin = lane < CH && c0 + lane < BD ? lane : 0;
    const float xf0 = wave == 0 ? p.xin[(size_t)((cb + 1) & 1) * BD + c0 + jin] : 0.f;
    const int logG = 31 - __clz(G);
    auto grow = [&](int rho) {                             // history row of local row rho
        return ((size_t)(rho % M) * BD + c0 + rho / M) * (size_t)p.L;
    };
    auto trow = [&](int rho) {                             // tap-table row
        return (size_t)(rho % M) * p.D + (c0 + rho / M) % p.D;
    };
    auto live = [&](int rho) { return c0 + rho / M < BD; };

    // helper lanes: row hrho, taps h[seg + 8m] (zero for k < 2: the chain
    // adds tap 1, tap 0 is the red cell's own term); loads issued first
    // a helper wave holds 8 rows, each in lanes 4q..4q+3 (segments 0..3) and
    // 32+4q..+3 (segments 4..7): every half-wave then reads 8 rows x 4
    // segments, 32 distinct banks (slot width 8 mod 32)
    const int hw = (wave & 3) ? wave - 1 - wave / 4 : -1;
    const int hrho = hw * (kLanes / S) + ((lane >> 2) & 7);
    const int seg = (lane & 3) | ((lane >> 5) << 2);
    const bool helper = hw >= 0 && hrho < R && live(hrho);
    float hreg[kChunkTaps];
    // the lane's 32 taps lie together in the tap table: eight 16-byte loads,
    // of which a chunk of G positions needs the first G/32 (taps 4q..4q+3 of
    // a lane are lags seg + 32q + 8j, all at least G from q = G/32 on).  The
    // groups used from the first position on (q < 2: lags below 64; the
    // pushed taps) are loaded here; the later pulled groups after the set-up's
    // loads, so that the set-up does not wait for them: their first use is at
    // position 62.  No mask waits for a load either: the table holds zeros at
    // lags 0 and 1, a lane without a helper row discards its sums, and a
    // group is loaded only when its lags lie in the chunk, but for the one
    // group of chunks shorter than 32, whose lags past the chunk are zeroed.
    constexpr int QP = kChunkPullTaps / 4;                 // groups q >= QP are pushed
    const float4 *tp = (const float4 *)(p.htap + (size_t)(helper ? trow(hrho) : 0) * kChunkTapRow +
                                        seg * kChunkTaps);
    auto tap_group = [&](int q) {
        const float4 v = 32 * q < G ? tp[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        hreg[4 * q] = v.x;
        hreg[4 * q + 1] = v.y;
        hreg[4 * q + 2] = v.z;
        hreg[4 * q + 3] = v.w;
    };
    if (hw >= 0) {
#pragma unroll
        for (int q = 0; q < kChunkTaps / 4; ++q)
            if (q < 2 || q >= QP) tap_group(q);
        if (G < 32) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (seg + S * m >= G) hreg[m] = 0.f;
        }
    }

    // Set-up by waves 1..15: the pending sums of the chunk's positions (rows
    // of the history, G slots each), the heads, the zero rows, the
    // teacher-forced inputs.
    const int pt = threadIdx.x - kLanes, npt = blockDim.x - kLanes;
    if (wave > 0) {
        // the heads, one row per thread (R <= kChunkMaxRows < npt), in flight
        // together with the pending sums
        float2 hv = make_float2(0.f, 0.f);
        if (pt < R && live(pt)) {
            const int l = pt % M, c = (c0 + pt / M) % p.D;   // from the heads table: 8 rows per line
            hv = make_float2(p.hh[head(p, l, 0, c)], p.HK > 1 ? p.hh[head(p, l, 1, c)] : 0.f);
        }
        if (G >= 16) {
            // Items of 16 rows x 4 float4 per wave: the loads read 64
            // contiguous bytes of each of 16 rows, and the stores (four slots
            // per float4; the items of one row lie 4 kChunkSlot floats apart,
            // on one bank) meet at most four lanes per bank, where an item
            // per row-major lane would put all 64 lanes of a store on one
            // bank.  A thread's loads all go out before its first store.
            constexpr int NB = 8, RW = 16, KW = 4;
            const int rg = (R + RW - 1) / RW;              // groups of 16 rows
            const int total = rg * (G >> 2) * RW;          // items, padded to whole row groups
            for (int e0 = pt; e0 < total; e0 += NB * npt) {
                float4 v[NB];
                int rho[NB], s0[NB];
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int e = e0 + k * npt;
                    const int blk = e >> 6, ln = e & 63;
                    rho[k] = (blk % rg) * RW + (ln & (RW - 1));
                    s0[k] = ((blk / rg) * KW + (ln >> 4)) * 4;
                    v[k] = e < total && rho[k] < R && live(rho[k])
                               ? *(const float4 *)(p.buf + grow(rho[k]) + cb + s0[k])
                               : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int e = e0 + k * npt;
                    if (e >= total) break;
                    if (rho[k] >= R) continue;
                    float *d = xp + (size_t)(G - 1 - s0[k]) * SP + rho[k];
                    d[0] = v[k].x;
                    d[-SP] = v[k].y;
                    d[-2 * SP] = v[k].z;
                    d[-3 * SP] = v[k].w;
                }
            }
        } else {
            for (int e = pt; e < R * G; e += npt) {
                const int rho = e >> logG;
                xp[(size_t)(G - 1 - (e & (G - 1))) * SP + rho] = live(rho) ? p.buf[grow(rho) + cb + (e & (G - 1))] : 0.f;
            }
        }
        for (int e = pt; e < kChunkZeroRows * SP; e += npt) xz[e] = 0.f;
        if (pt < R) h01[pt] = hv;
        if (xseq)
            for (int e = pt; e < G * CH; e += npt) {
                const int i = e / CH, j = e % CH;
                xs[e] = c0 + j < BD ? xseq[(size_t)i * BD + c0 + j] : 0.f;
            }
    }
    // every load so far is in, on every path (so that no use of the early
    // groups waits for the groups loaded next)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (hw >= 0) {
#pragma unroll
        for (int q = 2; q < QP; ++q) tap_group(q);
    }
    __syncthreads();

    float *hist = p.buf + (helper ? grow(hrho) + cb : 0);   // a helper row's positions of the chunk
    if (wave == 0) {
        // ---- red cells; the helpers do not share this wave's SIMD
        __builtin_amdgcn_s_setprio(3);
        chain_run<MT, (MODE & kChunkRec) != 0, (MODE & kChunkTanh) != 0>(
            p, xp, G, h01, cb, lane, c0 + lane, lane < CH && c0 + lane < BD, xseq ? xs : nullptr, CH, xf0);
    } else if (hw < 0) {
        // ---- waves 4, 8, 12: barriers only.  Wave 4 of the first and of the
        // last workgroup in dispatch order stamps each position's end, into
        // the stamps and their second row; the reader takes the later of the
        // two.  (An atomic maximum from every workgroup puts a hundred and
        // more atomics on one address per position, which the memory side
        // serialises: their backlog stalled whole positions.)
        const bool first_wg = blockIdx.x == 0, last_wg = blockIdx.x == gridDim.x - 1;
        long long *sp = p.stamps + (first_wg ? 0 : p.L + 1) + cb + 1;
        for (int i = 0; i < G; ++i) {
            __syncthreads();
            if (wave == 4 && lane == 0 && (first_wg || last_wg)) sp[i] = (long long)wall_clock64();
        }
    } else if (hw * (kLanes / S) >= R) {
        // ---- helper waves without a row (fewer rows than helper lanes):
        // barriers only, so they take no LDS or VALU time from the others
        for (int i = 0; i < G; ++i) __syncthreads();
    } else {
        // ---- helpers, during position i.  Pull: the pending sum of slot i+1
        // but for its tap-1 term, over lags 2 .. K-1 (K = 8 kChunkPullTaps):
        // fft + sum h[k] x_{i+1-k} (the pushes below have added the lags from
        // K on by then).  Tap m of a lane (k = seg + 8m) reads slot i+1-k at
        // row row0 + 8m; taps come in groups of eight m, a new group from
        // i = 62, 126, ... on (its other lanes then read the zero rows past
        // the chunk's first slot).  Push (chunks longer than K): the source
        // x_{i-1}, now final, times lags K .. 255 into the targets
        // i-1+K .. 255.  Pulling every lag would leave position i with i taps
        // per row, the last positions of a chunk with 255; split this way the
        // pulled lags stop growing at K-1 and the pushed ones shrink as the
        // chunk proceeds (a push costs a read and a write per tap).
        auto position = [&](int i) {
            // every 32 positions, the inputs of the last 32 into the history,
            // for the FFT block at the chunk's end: one whole 128-byte line per
            // row, 16 bytes per lane (slots i-32+4seg .. +3, from row G-i+31-4seg down)
            if (helper && i >= 32 && (i & 31) == 0) {
                const float *src = xp + (size_t)(G - i + 31 - 4 * seg) * SP + hrho;
                *(float4 *)(hist + i - 32 + 4 * seg) = make_float4(src[0], src[-SP], src[-2 * SP], src[-3 * SP]);
            }
            if (i + 1 < G) {
                const int row0 = G - 2 - i + seg;
                float acc = 0.f;
                dispatch<kChunkPullTaps / 8 - 1>(min((i + 2) >> 6, kChunkPullTaps / 8 - 1), [&](auto nf) {
                    acc = helper_sum<decltype(nf)::value>(xp, hreg, row0, hrho, seg < 2);
                });
                acc = row_sum8(acc);
                if (helper && seg == 0) xp[(size_t)(G - 2 - i) * SP + hrho] += acc;
            }
            if (G > 8 * kChunkPullTaps && i >= 1 && i <= G - 8 * kChunkPullTaps && helper) {
                const float x = xp[(size_t)(G - i) * SP + hrho];             // slot i-1
                const int rowp = G - i - seg - 8 * kChunkPullTaps;             // target of the first pushed tap
                // pushed taps present in every lane of the wave: m <= (G-i-7)/8
                const int c = min(kChunkTaps - kChunkPullTaps, max(0, ((G - i - 7) >> 3) - kChunkPullTaps + 1));
                dispatch<kChunkTaps - kChunkPullTaps>(c, [&](auto cc) {
                    helper_push<decltype(cc)::value>(xp, hreg, rowp, hrho, x);
                });
            }
            __syncthreads();                   // the chain has written slot i
        };
        // the pulled groups q >= 2, loaded after the set-up, are first read at
        // position 62: one wait for them there (inside the loop it would also
        // wait for the history stores of the same position)
        const int i1 = min(G, 62);
        for (int i = 0; i < i1; ++i) position(i);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        for (int i = i1; i < G; ++i) position(i);
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

}  // namespace fi
