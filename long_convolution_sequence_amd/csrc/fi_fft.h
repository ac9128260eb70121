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
#include "fi_device.h"

namespace fi {

// One pad slot after every 16 complex values: strided accesses of late
// stages spread over the LDS banks.
__device__ __forceinline__ int lpad(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int lds_len(int n) { return n + (n >> 4); }

// W_S^j = exp(-2 pi i j / S), S = 2^slog, from the table of NT = 2^logNT roots.
__device__ __forceinline__ float2 twiddle(const float2 *__restrict__ tw, int logNT, int slog, int j) {
    return tw[j << (logNT - slog)];
}

// R radix-2 DIF stages on v[0..2^R).  The values sit at element offsets
// r + m*Q (Q = 2^qlog) of a block whose size at the first stage is 2^slog.
template <int R>
__device__ __forceinline__ void dif_stages(float2 (&v)[1 << R], int r, int slog, int qlog,
                                           const float2 *__restrict__ tw, int logNT) {
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int half = (1 << R) >> (t + 1);
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) {
            if ((m & half) == 0) {
                const int j = r + ((m & (half - 1)) << qlog);
                const float2 a = v[m], b = v[m + half];
                v[m] = cadd(a, b);
                v[m + half] = cmul(csub(a, b), twiddle(tw, logNT, slog - t, j));
            }
        }
    }
}

// Inverse of dif_stages up to a factor 2 per stage (conjugate twiddles,
// stages in reverse order).
template <int R>
__device__ __forceinline__ void dit_stages(float2 (&v)[1 << R], int r, int slog, int qlog,
                                           const float2 *__restrict__ tw, int logNT) {
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
        const int half = (1 << R) >> (t + 1);
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) {
            if ((m & half) == 0) {
                const int j = r + ((m & (half - 1)) << qlog);
                const float2 a = v[m];
                const float2 b = cmulc(v[m + half], twiddle(tw, logNT, slog - t, j));
                v[m] = cadd(a, b);
                v[m + half] = csub(a, b);
            }
        }
    }
}

// Compile-time description of a transform of 2^LOGN complex points.
template <int LOGN>
struct FftShape {
    static constexpr int N = 1 << LOGN;
    static constexpr int TT = N >= 16 ? N / 16 : 1;          // threads per transform
    static constexpr int TPB = TT >= 256 ? TT : 256;         // threads per block
    static constexpr int PER_BLOCK = TPB / TT;               // transforms per block
    static constexpr int R0 = LOGN < 4 ? LOGN : 4;           // stages of the outer group
    static constexpr int QLOG0 = LOGN - R0;
    static constexpr int HALF0 = (1 << R0) / 2;
    static constexpr int NPASS = (LOGN + 3) / 4;             // stage groups
    static constexpr int LDS = PER_BLOCK * lds_len(N);       // float2 per block
};

// Stage group PASS (>= 1) through LDS, all threads of one transform team.
template <int LOGN, int PASS, bool FWD>
__device__ __forceinline__ void lds_group(float2 *X, int lt, const float2 *__restrict__ tw, int logNT) {
    constexpr int SLOG = LOGN - 4 * PASS;
    constexpr int R = SLOG < 4 ? SLOG : 4;
    constexpr int QLOG = SLOG - R;
    constexpr int G = 1 << (LOGN - R);
    constexpr int TT = FftShape<LOGN>::TT;
    for (int g = lt; g < G; g += TT) {
        const int r = g & ((1 << QLOG) - 1);
        const int base = ((g >> QLOG) << SLOG) + r;
        float2 v[1 << R];
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) v[m] = X[lpad(base + (m << QLOG))];
        if (FWD)
            dif_stages<R>(v, r, SLOG, QLOG, tw, logNT);
        else
            dit_stages<R>(v, r, SLOG, QLOG, tw, logNT);
#pragma unroll
        for (int m = 0; m < (1 << R); ++m) X[lpad(base + (m << QLOG))] = v[m];
    }
}

// Forward stage groups 1 .. NPASS-1, each preceded by a block barrier.
template <int LOGN, int PASS>
__device__ __forceinline__ void forward_groups(float2 *X, int lt, const float2 *__restrict__ tw, int logNT) {
    if constexpr (PASS < FftShape<LOGN>::NPASS) {
        __syncthreads();
        lds_group<LOGN, PASS, true>(X, lt, tw, logNT);
        forward_groups<LOGN, PASS + 1>(X, lt, tw, logNT);
    }
}

// Inverse stage groups PASS, PASS-1, ..., 1, each followed by a block barrier.
template <int LOGN, int PASS>
__device__ __forceinline__ void inverse_groups(float2 *X, int lt, const float2 *__restrict__ tw, int logNT) {
    if constexpr (PASS >= 1) {
        lds_group<LOGN, PASS, false>(X, lt, tw, logNT);
        __syncthreads();
        inverse_groups<LOGN, PASS - 1>(X, lt, tw, logNT);
    }
}

template <int LOGN>
__device__ __forceinline__ int bitrev(int k) {
    return (int)(__brev((unsigned)k) >> (32 - LOGN));
}

// Real-spectrum pairing.  C holds the complex transform of c_k = a_{2k} + i a_{2k+1}
// (N points, bit-reversed positions).  For bin pair (k, N-k), with W = W_{2N}^k:
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
