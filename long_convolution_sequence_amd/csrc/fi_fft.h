// In-LDS complex FFT building blocks for the FFT gray-block kernels.
//
// Flash Inference (arXiv 2410.12982), summary page, Lemma 1 and
// "Zirkulaere Faltungs-Trick": the contribution of a block of U inputs to the
// next U outputs is a length-2U circular convolution whose upper half is
// exact.  Both sequences are real, so the 2U-point real transform is carried
// by a U-point complex transform of the even/odd-packed samples
// (c_k = a_{2k} + i a_{2k+1}), with the standard pairing of bins k and U-k to
// recover (and later re-pack) the real spectrum.
//
// Transform shape.  In-place radix-2 decimation in frequency (forward, natural
// order in, bit-reversed order out) and decimation in time (inverse,
// bit-reversed in, natural out), grouped four stages at a time: each thread
// holds 16 complex values in registers, runs four radix-2 stages on them and
// exchanges through LDS between groups.  Because the filter spectrum is
// multiplied in bit-reversed order, no permutation pass is ever needed.  The
// first forward group reads global memory directly (and skips the zero half of
// the padded input); the last inverse group writes only the wanted upper half
// straight into the accumulators.  Twiddles come from a table generated in
// fp64 on the host.
#pragma once
#include <type_traits>

#include "fi_device.h"

namespace fi {

// One pad slot after every 16 complex values: strided accesses of late
// stages spread over the LDS banks.
__device__ __forceinline__ int lpad(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int lds_len(int n) { return n + (n >> 4); }
// lpad(b + (m << q)) = lpad(b) + lpad_off(m, q) whenever b mod 16 plus
// (m << q) mod 16 stays below 16.  That holds for every access of a stage
// group (b its base, r < 2^q, the rest of b a multiple of 16 or of 2^(q+R))
// and of the outer group (b = lt): with m unrolled, each access then takes an
// immediate offset from one address instead of address arithmetic of its own.
__host__ __device__ constexpr int lpad_off(int m, int q) { return (m << q) + ((m << q) >> 4); }

// W_S^j = exp(-2 pi i j / S), S = 2^slog, from the table of NT = 2^logNT roots.
__device__ __forceinline__ float2 twiddle(const float2 *__restrict__ tw, int logNT, int slog, int j) {
    return tw[j << (logNT - slog)];
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// d * W_16^K and d * conj(W_16^K) for 0 <= K < 8 (W_16 = exp(-2 pi i / 16)).
constexpr float kC8 = 0.923879532511286756f;   // cos(pi/8)
constexpr float kS8 = 0.382683432365089772f;   // sin(pi/8)
constexpr float kR2 = 0.707106781186547524f;   // sqrt(2)/2
template <int K>
__device__ __forceinline__ float2 mul_w16(float2 d) {
    if constexpr (K == 0) return d;
    else if constexpr (K == 4) return make_float2(d.y, -d.x);
    else if constexpr (K == 2) return make_float2(kR2 * (d.x + d.y), kR2 * (d.y - d.x));
    else if constexpr (K == 6) return make_float2(kR2 * (d.y - d.x), -kR2 * (d.x + d.y));
    else {
        constexpr float c = K == 1 ? kC8 : K == 3 ? kS8 : K == 5 ? -kS8 : -kC8;
        constexpr float s = K == 1 ? kS8 : K == 3 ? kC8 : K == 5 ? kC8 : kS8;
        return make_float2(d.x * c + d.y * s, d.y * c - d.x * s);
    }
}
template <int K>
__device__ __forceinline__ float2 mul_w16c(float2 d) {
    if constexpr (K == 0) return d;
    else if constexpr (K == 4) return make_float2(-d.y, d.x);
    else if constexpr (K == 2) return make_float2(kR2 * (d.x - d.y), kR2 * (d.x + d.y));
    else if constexpr (K == 6) return make_float2(-kR2 * (d.x + d.y), kR2 * (d.x - d.y));
    else {
        constexpr float c = K == 1 ? kC8 : K == 3 ? kS8 : K == 5 ? -kS8 : -kC8;
        constexpr float s = K == 1 ? kS8 : K == 3 ? kC8 : K == 5 ? kC8 : kS8;
        return make_float2(d.x * c - d.y * s, d.y * c + d.x * s);
    }
}

// d * W_32^K and d * conj(W_32^K) for 0 <= K < 16 (W_32 = exp(-2 pi i / 32)).
constexpr float kCos16[9] = {1.f,
                             0.980785280403230449f,   // cos(pi/16)
                             0.923879532511286756f,   // cos(2 pi/16)
                             0.831469612302545237f,   // cos(3 pi/16)
                             0.707106781186547524f,   // cos(4 pi/16)
                             0.555570233019602225f,   // cos(5 pi/16)
                             0.382683432365089772f,   // cos(6 pi/16)
                             0.195090322016128268f,   // cos(7 pi/16)
                             0.f};
template <int K>
__device__ __forceinline__ float2 mul_w32(float2 d) {
    if constexpr (K % 2 == 0) return mul_w16<K / 2>(d);
    else {
        constexpr float c = K < 8 ? kCos16[K] : -kCos16[16 - K];  // cos(K pi / 16)
        constexpr float s = K < 8 ? kCos16[8 - K] : kCos16[K - 8];  // sin(K pi / 16)
        return make_float2(d.x * c + d.y * s, d.y * c - d.x * s);
    }
}
template <int K>
__device__ __forceinline__ float2 mul_w32c(float2 d) {
    if constexpr (K % 2 == 0) return mul_w16c<K / 2>(d);
    else {
        constexpr float c = K < 8 ? kCos16[K] : -kCos16[16 - K];
        constexpr float s = K < 8 ? kCos16[8 - K] : kCos16[K - 8];
        return make_float2(d.x * c - d.y * s, d.y * c + d.x * s);
    }
}

template <int R, int P>
constexpr int rev_bits() {
    int r = 0;
    for (int i = 0; i < R; ++i) r |= ((P >> i) & 1) << (R - 1 - i);
    return r;
}

// v[rev(k)] *= w^k (CONJ: conj(w)^k) for 0 < k < 2^R.  The powers come in
// order, w^k = w^(k-4) w^4 from k = 5 on, so at most five of them are live
// and none is more than five products away from w.
template <int R, bool CONJ>
__device__ __forceinline__ void apply_powers(float2 (&v)[1 << R], float2 w) {
    constexpr int NP = 1 << R;
    auto mul = [](float2 a, float2 b) { return CONJ ? cmulc(a, b) : cmul(a, b); };
    if constexpr (NP >= 2) {
        float2 pk[4];
        pk[1] = w;
        v[rev_bits<R, 1>()] = mul(v[rev_bits<R, 1>()], w);
        if constexpr (NP >= 4) {
            pk[2] = cmul(w, w);
            pk[3] = cmul(pk[2], w);
            v[rev_bits<R, 2>()] = mul(v[rev_bits<R, 2>()], pk[2]);
            v[rev_bits<R, 3>()] = mul(v[rev_bits<R, 3>()], pk[3]);
        }
        if constexpr (NP >= 8) {
            const float2 w4 = cmul(pk[2], pk[2]);
            pk[0] = w4;
            v[rev_bits<R, 4>()] = mul(v[rev_bits<R, 4>()], w4);
            static_for<5, NP>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                pk[k % 4] = cmul(pk[k % 4], w4);
                v[rev_bits<R, k>()] = mul(v[rev_bits<R, k>()], pk[k % 4]);
            });
        }
    }
}

// One group of R radix-2 DIF stages on v[0..2^R): the values sit at element
// offsets r + m*Q of a block of size S = 2^slog (Q = S / 2^R).  Equivalent
// form used here: a 2^R-point DFT over m with constant roots (output k left
// in register rev(k)), then the outer twiddle W_S^{r*k}.  PRUNED: the upper
// half of v is known to be zero.  TWIDDLE false: r is known to be 0 (the
// group spans a whole block), so the outer twiddles are all 1.
template <int R, bool PRUNED = false, bool TWIDDLE = true>
__device__ __forceinline__ void dif_group_w(float2 (&v)[1 << R], float2 w) {
    static_for<0, R>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int half = (1 << R) >> (t + 1);
        static_for<0, (1 << R)>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr ((m & half) == 0) {
                constexpr int k = (m & (half - 1)) * (16 / (2 * half));
                if constexpr (PRUNED && t == 0) {
                    v[m + half] = mul_w16<k>(v[m]);
                } else {
                    const float2 a = v[m], b = v[m + half];
                    v[m] = cadd(a, b);
                    v[m + half] = mul_w16<k>(csub(a, b));
                }
            }
        });
    });
    if constexpr (TWIDDLE) apply_powers<R, false>(v, w);
}
template <int R, bool PRUNED = false, bool TWIDDLE = true>
__device__ __forceinline__ void dif_group(float2 (&v)[1 << R], int r, int slog,
                                          const float2 *__restrict__ tw, int logNT) {
    dif_group_w<R, PRUNED, TWIDDLE>(v, TWIDDLE ? twiddle(tw, logNT, slog, r) : make_float2(1.f, 0.f));
}

// Inverse of dif_group up to the factor 2^R: conjugate outer twiddles, then
// the stages in reverse order with conjugate constant roots.
template <int R, bool TWIDDLE = true>
__device__ __forceinline__ void dit_group_w(float2 (&v)[1 << R], float2 w) {
    if constexpr (TWIDDLE) apply_powers<R, true>(v, w);
    static_for<0, R>([&](auto tc) {
        constexpr int t = R - 1 - decltype(tc)::value;
        constexpr int half = (1 << R) >> (t + 1);
        static_for<0, (1 << R)>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr ((m & half) == 0) {
                constexpr int k = (m & (half - 1)) * (16 / (2 * half));
                const float2 a = v[m];
                const float2 b = mul_w16c<k>(v[m + half]);
                v[m] = cadd(a, b);
                v[m + half] = csub(a, b);
            }
        });
    });
}
template <int R, bool TWIDDLE = true>
__device__ __forceinline__ void dit_group(float2 (&v)[1 << R], int r, int slog,
                                          const float2 *__restrict__ tw, int logNT) {
    dit_group_w<R, TWIDDLE>(v, TWIDDLE ? twiddle(tw, logNT, slog, r) : make_float2(1.f, 0.f));
}

// Compile-time description of a transform of 2^LOGN complex points.
template <int LOGN>
struct FftShape {
    static constexpr int N = 1 << LOGN;
    static constexpr int TT = N >= 16 ? N / 16 : 1;          // threads per transform
    // threads per block: one wave, or one transform when that is wider.
    // Measured in the pipeline against 256 threads: 2^7 points 10.2 against
    // 10.7 us, 2^8 16.6 against 17.4, 2^9 32.0 against 34.5, 2^10 61.7
    // against 65.6 us.
    static constexpr int TPB = TT > 64 ? TT : 64;
    static constexpr int PER_BLOCK = TPB / TT;               // transforms per block
    static constexpr int R0 = LOGN < 4 ? LOGN : 4;           // stages of the outer group
    static constexpr int QLOG0 = LOGN - R0;
    static constexpr int HALF0 = (1 << R0) / 2;
    static constexpr int NPASS = (LOGN + 3) / 4;             // stage groups
    static constexpr int LDS = PER_BLOCK * lds_len(N);       // float2 per block
};

// The outer twiddle root W_S^r of thread lt's group in stage group PASS
// (PASS >= 1: the LDS groups; PASS = 0: the outer group, S = 2^LOGN, r = lt).
// Every twiddled LDS group has four stages, so a thread owns exactly one
// group of it: the root can be read before the barrier that precedes the
// group, and its latency hides behind the barrier.
template <int LOGN, int PASS>
__device__ __forceinline__ float2 group_root(int lt, const float2 *__restrict__ tw, int logNT) {
    constexpr int SLOG = LOGN - 4 * PASS;
    constexpr int R = SLOG < 4 ? SLOG : 4;
    constexpr int QLOG = SLOG - R;
    if constexpr (PASS == 0) return twiddle(tw, logNT, LOGN, lt);
    else if constexpr (QLOG > 0) return twiddle(tw, logNT, SLOG, lt & ((1 << QLOG) - 1));
    else return make_float2(1.f, 0.f);
}

// Stage group PASS (>= 1) through LDS, all threads of one transform team; w is
// group_root<LOGN, PASS>.
template <int LOGN, int PASS, bool FWD>
__device__ __forceinline__ void lds_group(float2 *X, int lt, float2 w) {
    constexpr int SLOG = LOGN - 4 * PASS;
    constexpr int R = SLOG < 4 ? SLOG : 4;
    constexpr int QLOG = SLOG - R;
    constexpr int G = 1 << (LOGN - R);
    constexpr int TT = FftShape<LOGN>::TT;
    static_assert(QLOG == 0 || G == TT, "a twiddled group is the only one of its thread");
    for (int g = lt; g < G; g += TT) {
        const int r = g & ((1 << QLOG) - 1);
        float2 *Xb = X + lpad(((g >> QLOG) << SLOG) + r);
        float2 v[1 << R];
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) v[m] = Xb[lpad_off(m, QLOG)];
        if constexpr (FWD)
            dif_group_w<R, false, (QLOG > 0)>(v, w);
        else
            dit_group_w<R, (QLOG > 0)>(v, w);
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) Xb[lpad_off(m, QLOG)] = v[m];
    }
}

// Forward stage groups PASS .. END-1 (by default through NPASS-1), each
// preceded by a block barrier.  PRE: each group's root is read before its
// barrier (off where the registers it holds across the barrier would spill).
template <int LOGN, int PASS, int END = FftShape<LOGN>::NPASS, bool PRE = true>
__device__ __forceinline__ void forward_groups(float2 *X, int lt, const float2 *__restrict__ tw, int logNT) {
    if constexpr (PASS < END) {
        if constexpr (PRE) {
            const float2 w = group_root<LOGN, PASS>(lt, tw, logNT);
            __syncthreads();
            lds_group<LOGN, PASS, true>(X, lt, w);
        } else {
            __syncthreads();
            lds_group<LOGN, PASS, true>(X, lt, group_root<LOGN, PASS>(lt, tw, logNT));
        }
        forward_groups<LOGN, PASS + 1, END, PRE>(X, lt, tw, logNT);
    }
}

// Inverse stage groups PASS, PASS-1, ..., 1, each followed by a block barrier;
// w = group_root<LOGN, PASS> (PRE: read by the caller before its barrier, and
// each next root read here before the barrier; otherwise w is not used and
// every root is read after the barrier).  Returns group_root<LOGN, 0>, the
// root of the outer group that follows.
template <int LOGN, int PASS, bool PRE = true>
__device__ __forceinline__ float2 inverse_groups(float2 *X, int lt, const float2 *__restrict__ tw, int logNT,
                                                 float2 w) {
    if constexpr (PASS >= 1) {
        if constexpr (PRE) {
            lds_group<LOGN, PASS, false>(X, lt, w);
            const float2 wn = group_root<LOGN, PASS - 1>(lt, tw, logNT);
            __syncthreads();
            return inverse_groups<LOGN, PASS - 1, PRE>(X, lt, tw, logNT, wn);
        } else {
            lds_group<LOGN, PASS, false>(X, lt, group_root<LOGN, PASS>(lt, tw, logNT));
            __syncthreads();
            return inverse_groups<LOGN, PASS - 1, PRE>(X, lt, tw, logNT, w);
        }
    } else {
        return PRE ? w : group_root<LOGN, 0>(lt, tw, logNT);
    }
}

// Bit reversal of the low w bits of k (1 <= w <= 31), for host and device.
__host__ __device__ constexpr unsigned brev32(unsigned v) {
    v = ((v >> 1) & 0x55555555u) | ((v & 0x55555555u) << 1);
    v = ((v >> 2) & 0x33333333u) | ((v & 0x33333333u) << 2);
    v = ((v >> 4) & 0x0f0f0f0fu) | ((v & 0x0f0f0f0fu) << 4);
    v = ((v >> 8) & 0x00ff00ffu) | ((v & 0x00ff00ffu) << 8);
    return (v >> 16) | (v << 16);
}
__host__ __device__ constexpr int rbits(int w, int k) { return (int)(brev32((unsigned)k) >> (32 - w)); }

// Work items of the real-spectrum step.  Bins k and N-k of the complex
// transform are combined; they sit at the bit-reversed positions
// rev(k), rev(N-k).  Item e in [0, N/2) names one such pair:
//   pj: position of bin j (0 <= j < N/2), pm: position of bin N-j.
// Item 0 is special: bins 0 and N/2, both self-paired (positions 0 and 1).
// For N >= 32 the items run over 16-position groups so that sixteen
// consecutive items touch sixteen consecutive positions (and the reversed
// run of the partner group), which keeps the LDS accesses of a wave free of
// bank conflicts: with k = a*(N/16) + b (a = rev4 of the position's low four
// bits, b = rev of its group index), bin N-k lies in group rev(N/16 - b) at
// offset 15 - (low bits).  Items 0..7: group 0 (pairs a <-> 16-a);
// 8..15: group rev(N/32) = 1 (self-partnered, offsets i <-> 15-i);
// 16..: group pairs b <-> N/16 - b for 1 <= b < N/32.
struct PairSlot {
    int pj, pm, j;
};
__host__ __device__ inline PairSlot pair_slot(int logn, int e) {
    const int N = 1 << logn;
    if (e == 0) return {0, 1, 0};
    int p1, p2;
    if (logn <= 4) {
        p1 = rbits(logn, e);
        p2 = rbits(logn, N - e);
    } else if (e < 8) {
        p1 = rbits(4, e);
        p2 = rbits(4, 16 - e);
    } else if (e < 16) {
        p1 = 16 + (e - 8);
        p2 = 31 - (e - 8);
    } else {
        const int b = ((e - 16) >> 4) + 1, i = e & 15;
        p1 = 16 * rbits(logn - 4, b) + i;
        p2 = 16 * rbits(logn - 4, (N >> 4) - b) + 15 - i;
    }
    const int k1 = rbits(logn, p1);
    if (k1 < N / 2) return {p1, p2, k1};
    return {p2, p1, N - k1};
}

// pair_slot of the items e = lt + m*TT of one thread (TT = N/16 >= 16, so
// N >= 256; m < 8) as a part fixed per thread plus a part that depends on m
// alone, so that with m unrolled the slots cost no arithmetic per item.  For
// e >= 16, e >> 4 = (lt >> 4) + m*2^(w-4) (w = log2 N - 4): its w-bit
// reversal is rev(lt >> 4) << 4 | rev4(m), and 2^w - (e >> 4) has the high
// four bits 15 - m over the low part 2^(w-4) - (lt >> 4) when lt >> 4 > 0,
// or 16 - m over zero when lt < 16.  Which of the pair comes first is bit 0
// of p1 (the top bit of its bin), i = lt & 15 for every m.  Item m = 0 of the
// threads lt < 16 has e < 16: the caller takes pair_slot there.
struct PairBase {
    int p1, p2;      // per-thread parts of the two slots
    bool lo, swap;   // lt >= 16; the bin of p1 is in the upper half
};
template <int LOGN>
__host__ __device__ inline PairBase pair_base(int lt) {
    static_assert(LOGN >= 8, "sixteen or more threads per transform");
    constexpr int W4 = LOGN - 8;   // bits of lt >> 4
    const int bl = lt >> 4, i = lt & 15;
    const int r1 = W4 > 0 ? rbits(W4, bl) : 0;
    const int r2 = (W4 > 0 && bl > 0) ? rbits(W4, (1 << W4) - bl) : 0;
    return {256 * r1 + i, 256 * r2 + 15 - i, bl > 0, (i & 1) != 0};
}
template <int LOGN>
__host__ __device__ inline PairSlot pair_slot_m(const PairBase &b, int m) {
    const int p1 = b.p1 + 16 * rbits(4, m);
    const int p2 = b.p2 + 16 * (b.lo ? rbits(4, 15 - m) : rbits(4, 16 - m));
    return b.swap ? PairSlot{p2, p1, 0} : PairSlot{p1, p2, 0};
}

// LDS slots (lpad applied) of the pair of item e = lt + m*TT: a = bin j,
// b = bin N - j.  From N = 256 on, the per-thread parts are padded once
// (lpad(x + 16c) = lpad(x) + 17c) and an item adds compile-time constants.
struct SlotPair {
    int a, b;
};
struct PairLds {
    int l1, l2;
    bool lo, swap;
};
template <int LOGN>
__host__ __device__ inline PairLds pair_lds(int lt) {
    if constexpr (LOGN >= 8) {
        const PairBase b = pair_base<LOGN>(lt);
        return {lpad(b.p1), lpad(b.p2), b.lo, b.swap};
    } else {
        return {0, 0, false, false};
    }
}
template <int LOGN, int TT>
__host__ __device__ inline SlotPair item_lds(const PairLds &b, int lt, int m) {
    if constexpr (LOGN >= 8) {
        const int s1 = b.l1 + 17 * rbits(4, m);
        const int s2 = b.l2 + 17 * (b.lo ? rbits(4, 15 - m) : rbits(4, 16 - m));
        const SlotPair f = b.swap ? SlotPair{s2, s1} : SlotPair{s1, s2};
        if (m != 0) return f;
        // item 0 of the threads lt < 16 (e = lt < 16) follows the first groups' order
        const PairSlot ps = pair_slot(LOGN, lt);
        return lt < 16 ? SlotPair{lpad(ps.pj), lpad(ps.pm)} : f;
    } else {
        const PairSlot ps = pair_slot(LOGN, lt + m * TT);
        return {lpad(ps.pj), lpad(ps.pm)};
    }
}

// Transforms of N = 2M points done as two M-point halves.  The first radix-2
// stage of a decimation in frequency splits the bins by parity: the even bins
// are the M-point transform of (c_lo + c_hi), the odd bins that of
// (c_lo - c_hi) W_N^m.  Bin k pairs with N-k, which has the same parity, so
// each half keeps its own real-spectrum step.  In the even half, bin 2j is
// bin j of an M-point transform and pairs as in pair_slot (with
// W_{2N}^{2j} = W_{2M}^j).  In the odd half, bin 2k'+1 pairs with
// 2(M-1-k')+1, and rev(M-1-k') = M-1-rev(k'): positions p and M-1-p.  Item
// e in [0, M/2) takes the even position 2e (its bin k' = rev(2e) is below M/2)
// and its mirror M-1-2e; sixteen consecutive items touch sixteen distinct LDS
// bank slots.  odd_slot(e).j is the bin 2k'+1 of the N-point transform.
__host__ __device__ inline PairSlot odd_slot(int logm, int e) {
    const int M = 1 << logm;
    return {2 * e, M - 1 - 2 * e, 2 * rbits(logm, 2 * e) + 1};
}

// Real-spectrum pairing.  C holds the complex transform of c_k = a_{2k} + i a_{2k+1}
// (N points, bit-reversed positions, see pair_slot).  For bin pair (k, N-k), with W = W_{2N}^k:
//   E = (C_k + conj C_{N-k})/2,  O = (C_k - conj C_{N-k})/(2i)
//   A_k = E + W O,  A_{N-k} = conj(E - W O)          (bins of the 2N-point real FFT)
// and the inverse packing of a real spectrum Z into D (so that the inverse
// N-point transform of D gives z_{2m} + i z_{2m+1}):
//   Ze = (Z_k + conj Z_{N-k})/2,  Zo = (Z_k - conj Z_{N-k}) conj(W)/2
//   D_k = Ze + i Zo,  D_{N-k} = conj(Ze) + i conj(Zo).
__device__ __forceinline__ void real_bins(float2 C1, float2 C2, float2 W, float2 &A1, float2 &A2) {
    const float2 E = make_float2(0.5f * (C1.x + C2.x), 0.5f * (C1.y - C2.y));
    const float2 O = make_float2(0.5f * (C1.y + C2.y), -0.5f * (C1.x - C2.x));
    const float2 WO = cmul(W, O);
    A1 = cadd(E, WO);
    const float2 d = csub(E, WO);
    A2 = make_float2(d.x, -d.y);
}

__device__ __forceinline__ void pack_inverse(float2 Z1, float2 Z2, float2 W, float2 &D1, float2 &D2) {
    const float2 Ze = make_float2(0.5f * (Z1.x + Z2.x), 0.5f * (Z1.y - Z2.y));
    const float2 Zo = cmulc(make_float2(0.5f * (Z1.x - Z2.x), 0.5f * (Z1.y + Z2.y)), W);
    D1 = make_float2(Ze.x - Zo.y, Ze.y + Zo.x);
    D2 = make_float2(Ze.x + Zo.y, -Ze.y + Zo.x);
}

}  // namespace fi
