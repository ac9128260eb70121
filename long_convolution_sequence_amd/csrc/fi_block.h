// Hyena-style block between mixer layers (18-layer B=4 D=768 block workload).
//
// Flash Inference (arXiv 2410.12982), summary page, "Modellarchitektur": each
// layer is mixer then block, a^l = block^l(mixer^l(a^{l-1})); "Experimentelle
// Einrichtung": the blocks are an MLP with GELU in the synthetic setting and
// Hyena's in the real one.  The pages do not define Hyena's internals; the
// reading implemented here (and in the CPU oracle, separately):
//   [u | v | w] = x W          (W: D x 3D, column thirds)
//   q = u * w                  the layer's convolution input (red cell, tiles)
//   c = pending + h0 * q       the mixer output (red cell)
//   m = v * c
//   z = GELU(m W1) W2          (W1: D x 4D, W2: 4D x D, exact-erf GELU, no bias)
//   a = z / sqrt(mean(z^2) + 1e-6)   (RMSNorm, unit gain, no residual)
// and the next position's layer-0 input is tanh(a^{M-1}).
//
// Weights are bf16, stored transposed ([N][K], rows contiguous in k) so that
// one wave reads one output's weight row with coalesced loads; activations are
// fp32 and each wave keeps its slice of them in registers (see the GEMVs
// below).  The GEMVs have B <= 8 rows: they are HBM/L2-bound matrix-vector
// products, not dense contractions, so they run on the vector ALUs.
#pragma once
#include "fi_device.h"

namespace fi {

constexpr int kBlockMaxB = 8;
constexpr float kRmsEps = 1e-6f;

__device__ __forceinline__ float bf16f(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// The GEMVs: one wave covers a stretch of K = up to kBlockSpan values of the
// input rows, lane l the values k = 256 j + 4 l .. +3 for j < kBlockChunks, so
// each weight load (four bf16, 8 bytes) of a wave reads 512 contiguous bytes
// and each input load is a float4.  The wave keeps its inputs (B rows) in
// registers and runs them against R weight rows; a row's partial sums over
// the wave's k then meet in a butterfly of shuffles.  Each weight row is read
// by one wave (or, for the down projection, each quarter of it by one wave of
// the workgroup); so every weight byte is read once per position, with all of
// a matrix's loads in flight at once.
constexpr int kBlockChunks = 3;                     // 256-value chunks per wave
constexpr int kBlockSpan = 256 * kBlockChunks;      // K covered by one wave (768)
constexpr int kBlockRows = 2;                        // weight rows per wave (up and down projections)

template <int B>
struct WaveIn {                                      // a wave's slice of B input rows
    float4 v[kBlockChunks][B];
};

// Load rows src[b][k0 + k] (row stride ld, k < K) of this lane's slice; scale[b]
// multiplies row b when given; values past K are zero.
template <int B>
__device__ __forceinline__ void load_in(WaveIn<B> &in, const float *src, int ld, int k0, int K, const float *scale,
                                        int lane) {
#pragma unroll
    for (int j = 0; j < kBlockChunks; ++j) {
        const int k = 256 * j + 4 * lane;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float4 v = k < K ? *reinterpret_cast<const float4 *>(src + (size_t)b * ld + k0 + k)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
            if (scale) {
                const float sc = scale[b];
                v = make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc);
            }
            in.v[j][b] = v;
        }
    }
}

// out[b] = sum over the wave's slice of wrow[k] * in[b][k] (wrow already offset
// to the slice), summed over the wave: the full value lands in every lane.
template <int B>
__device__ __forceinline__ void wave_dot(const unsigned short *__restrict__ wrow, const WaveIn<B> &in, int K,
                                         int lane, float (&out)[B]) {
    uint2 q[kBlockChunks];
#pragma unroll
    for (int j = 0; j < kBlockChunks; ++j) {
        const int k = 256 * j + 4 * lane;
        q[j] = k < K ? *reinterpret_cast<const uint2 *>(wrow + k) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) out[b] = 0.f;
#pragma unroll
    for (int j = 0; j < kBlockChunks; ++j) {
        const float w0 = __uint_as_float(q[j].x << 16), w1 = __uint_as_float(q[j].x & 0xffff0000u);
        const float w2 = __uint_as_float(q[j].y << 16), w3 = __uint_as_float(q[j].y & 0xffff0000u);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float4 x = in.v[j][b];
            out[b] = fmaf(w0, x.x, fmaf(w1, x.y, fmaf(w2, x.z, fmaf(w3, x.w, out[b]))));
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) out[b] = wave_sum(out[b]);
}

// Layer l, step 1: the layer input (x^0 for l = 0, else RMSNorm of the
// previous layer's z, its norm taken by each wave from its own copy of z),
// the projection rows of channel c (u, v, w), the gate and the red cell.  One
// wave per channel, four per workgroup.
template <int B>
__global__ void __launch_bounds__(256) k_hy_proj(Dev p, int rd, int l, const float *xext) {
    const long long n = position_of(p, rd);
    if (n > p.L) return;                           // uniform guard
    const int D = p.D, BD = B * D;
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= D) return;                            // no barrier below
    // the red cell's head and pending sum (lane b: chain b*D + c), read first so
    // that their latency passes under the input and weight loads
    const size_t rcell = ring(p, n, l) + (size_t)(lane < B ? lane : 0) * D + c;
    const float h0 = p.hh[head(p, l, 0, c)];
    const float pend = lane < B ? p.ar[rcell] : 0.f;
    WaveIn<B> in;
    if (l == 0) {
        load_in<B>(in, xext ? xext : p.xin + (size_t)(n & 1) * BD, D, 0, D, nullptr, lane);
    } else {
        load_in<B>(in, p.zb, D, 0, D, nullptr, lane);
        float rs[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < kBlockChunks; ++j) {
                const float4 v = in.v[j][b];
                ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
            }
            rs[b] = 1.0f / sqrtf(wave_sum(ss) / (float)D + kRmsEps);
        }
#pragma unroll
        for (int j = 0; j < kBlockChunks; ++j)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float4 v = in.v[j][b];
                in.v[j][b] = make_float4(v.x * rs[b], v.y * rs[b], v.z * rs[b], v.w * rs[b]);
            }
        if (p.reca && c == 0) {                    // the previous layer's block output a = z / rms
#pragma unroll
            for (int j = 0; j < kBlockChunks; ++j) {
                const int k = 256 * j + 4 * lane;
                if (k < D)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        *reinterpret_cast<float4 *>(p.reca + ((size_t)(n - 1) * p.M + (l - 1)) * BD + b * D + k) =
                            in.v[j][b];
            }
        }
    }
    const unsigned short *W = p.Wt + (size_t)l * 3 * D * D;
    float u[B], v[B], w[B];
    wave_dot<B>(W + (size_t)c * D, in, D, lane, u);
    wave_dot<B>(W + (size_t)(D + c) * D, in, D, lane, v);
    wave_dot<B>(W + (size_t)(2 * D + c) * D, in, D, lane, w);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        if (lane == b) {
            const int chain = b * D + c;
            const size_t r = rcell;
            const float q = u[b] * w[b];
            const float cv = fmaf(h0, q, pend);
            p.xr[r] = q;
            if (p.recx) {
                const size_t rr = ((size_t)(n - 1) * p.M + l) * BD + chain;
                p.recx[rr] = q;
                p.recy[rr] = cv;
            }
            p.mb[chain] = v[b] * cv;
        }
    }
}

// Layer l, step 2: hidden = GELU(m W1), kBlockRows hidden units per wave.
template <int B>
__global__ void __launch_bounds__(256) k_hy_up(Dev p, int rd, int l) {
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int D = p.D;
    const int lane = threadIdx.x & 63;
    const int j0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kBlockRows;
    if (j0 >= 4 * D) return;
    WaveIn<B> in;
    load_in<B>(in, p.mb, D, 0, D, nullptr, lane);
#pragma unroll
    for (int r = 0; r < kBlockRows; ++r) {
        const int j = j0 + r;
        if (j >= 4 * D) break;
        float s[B];
        wave_dot<B>(p.W1t + ((size_t)l * 4 * D + j) * D, in, D, lane, s);
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (lane == b) p.hb[(size_t)b * 4 * D + j] = 0.5f * s[b] * (1.0f + erff(s[b] * 0.70710678118654752f));
    }
}

// Layer l, step 3: z = hidden W2.  A workgroup owns kBlockRows output channels;
// its four waves take the four quarters of the hidden units (D each) and their
// partial sums meet in LDS.
template <int B>
__global__ void __launch_bounds__(256) k_hy_down(Dev p, int rd, int l) {
    __shared__ float part[4][kBlockRows][B];
    const long long n = position_of(p, rd);
    if (n > p.L) return;                           // uniform guard
    const int D = p.D;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * kBlockRows;
    WaveIn<B> in;
    load_in<B>(in, p.hb, 4 * D, wave * D, D, nullptr, lane);
#pragma unroll
    for (int r = 0; r < kBlockRows; ++r) {
        const int c = c0 + r;
        float s[B];
        if (c < D) {
            wave_dot<B>(p.W2t + ((size_t)l * D + c) * 4 * D + (size_t)wave * D, in, D, lane, s);
        } else {
#pragma unroll
            for (int b = 0; b < B; ++b) s[b] = 0.f;
        }
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (lane == b) part[wave][r][b] = s[b];
    }
    __syncthreads();
    if (threadIdx.x < kBlockRows * B) {
        const int r = threadIdx.x / B, b = threadIdx.x % B;
        const int c = c0 + r;
        if (c < D) p.zb[(size_t)b * D + c] = (part[0][r][b] + part[1][r][b]) + (part[2][r][b] + part[3][r][b]);
    }
}

// 1 / sqrt(mean(z[b]^2) + eps) for every row, into rs[b] (LDS).  One wave per row.
__device__ __forceinline__ void row_rms(const float *z, float *rs, int B, int D) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
    for (int b = wave; b < B; b += waves) {
        float s = 0.f;
        for (int k = lane; k < D; k += 64) s = fmaf(z[b * D + k], z[b * D + k], s);
        s = wave_sum(s);
        if (lane == 0) rs[b] = 1.0f / sqrtf(s / (float)D + kRmsEps);
    }
}

// After the last layer: a^{M-1} = RMSNorm(z); output, record, next input tanh(a).
// Each workgroup takes its stretch of the B*D outputs (and forms every row's
// norm itself: B*D values, far less than the outputs' own latency).
static __global__ void __launch_bounds__(256) k_hy_out(Dev p, int rd, float *yext) {
    __shared__ float rs[kBlockMaxB];
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int B = p.B, D = p.D, BD = B * D;
    row_rms(p.zb, rs, B, D);
    __syncthreads();
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < BD; i += gridDim.x * blockDim.x) {
        const float a = p.zb[i] * rs[i / D];
        p.ylast[(size_t)(n - 1) * BD + i] = a;
        if (yext) yext[i] = a;
        if (p.reca) p.reca[((size_t)(n - 1) * p.M + (p.M - 1)) * BD + i] = a;
        p.xin[(size_t)((n + 1) & 1) * BD + i] = apply_map(p.fb, a);
    }
}

// dst[c][r] = src[r][c] for a rows x cols matrix of 16-bit values.
static __global__ void __launch_bounds__(256) k_transpose16(const unsigned short *src, unsigned short *dst, int rows,
                                                     int cols) {
    __shared__ unsigned short t[32][33];
    const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (int i = ty; i < 32; i += 8) {
        const int r = by + i, c = bx + tx;
        if (r < rows && c < cols) t[i][tx] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int c = bx + i, r = by + tx;
        if (r < rows && c < cols) dst[(size_t)c * rows + r] = t[tx][i];
    }
}

}  // namespace fi
