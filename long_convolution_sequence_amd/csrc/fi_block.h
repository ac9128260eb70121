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
// one wave reads one output's weight row with 16-byte loads; activations are
// fp32 and staged in LDS in a swizzled order (k = 8*c8 + e at e*(K/8) + c8)
// so that lane c8's eight reads of a chunk hit eight distinct banks.
// The GEMVs have B <= 8 rows: they are HBM/L2-bound matrix-vector products,
// not dense contractions, so they run on the vector ALUs.
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

// Stage rows src[b][0..K) (scaled by scale[b]) into xs in swizzled order.
__device__ __forceinline__ void stage_rows(float *xs, const float *src, const float *scale, int B, int K) {
    const int C8 = K / 8;
    for (int i = threadIdx.x; i < B * K; i += blockDim.x) {
        const int b = i / K, k = i % K;
        const float v = src[i] * (scale ? scale[b] : 1.f);
        xs[b * K + (k % 8) * C8 + k / 8] = v;
    }
}

// out[b] = sum_k wrow[k] * x[b][k] over the staged rows; the full sum lands in
// every lane.  K is a multiple of 8.
__device__ __forceinline__ void row_dot(const unsigned short *__restrict__ wrow, const float *xs, int B, int K,
                                        int lane, float (&out)[kBlockMaxB]) {
    const int C8 = K / 8;
    float acc[kBlockMaxB];
#pragma unroll
    for (int b = 0; b < kBlockMaxB; ++b) acc[b] = 0.f;
#pragma unroll 2
    for (int c8 = lane; c8 < C8; c8 += 64) {
        const uint4 q = *reinterpret_cast<const uint4 *>(wrow + 8 * c8);
        float w[8];
        w[0] = __uint_as_float(q.x << 16); w[1] = __uint_as_float(q.x & 0xffff0000u);
        w[2] = __uint_as_float(q.y << 16); w[3] = __uint_as_float(q.y & 0xffff0000u);
        w[4] = __uint_as_float(q.z << 16); w[5] = __uint_as_float(q.z & 0xffff0000u);
        w[6] = __uint_as_float(q.w << 16); w[7] = __uint_as_float(q.w & 0xffff0000u);
#pragma unroll
        for (int b = 0; b < kBlockMaxB; ++b) {
            if (b < B) {
                const float *xb = xs + b * K + c8;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[b] = fmaf(w[e], xb[e * C8], acc[b]);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < kBlockMaxB; ++b) out[b] = b < B ? wave_sum(acc[b]) : 0.f;
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

// Layer l, step 1: layer input (x^0 for l = 0, else RMSNorm of the previous
// layer's z), projection, gate, red cell.  Block = 4 waves = 4 channels.
__global__ void __launch_bounds__(256) k_hy_proj(Dev p, int rd, int l, const float *xext) {
    extern __shared__ float xs[];                  // [B][D] swizzled
    __shared__ float rs[kBlockMaxB];
    const long long n = position_of(p, rd);
    if (n > p.L) return;                           // uniform guard
    const int B = p.B, D = p.D, BD = B * D;
    const float *src;
    if (l == 0) {
        src = xext ? xext : p.xin + (size_t)(n & 1) * BD;
    } else {
        row_rms(p.zb, rs, B, D);
        __syncthreads();
        src = p.zb;
        if (p.reca && blockIdx.x == 0) {
            for (int i = threadIdx.x; i < BD; i += blockDim.x)
                p.reca[((size_t)(n - 1) * p.M + (l - 1)) * BD + i] = p.zb[i] * rs[i / D];
        }
    }
    stage_rows(xs, src, l == 0 ? nullptr : rs, B, D);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= D) return;
    const unsigned short *W = p.Wt + (size_t)l * 3 * D * D;
    float u[kBlockMaxB], v[kBlockMaxB], w[kBlockMaxB];
    row_dot(W + (size_t)c * D, xs, B, D, lane, u);
    row_dot(W + (size_t)(D + c) * D, xs, B, D, lane, v);
    row_dot(W + (size_t)(2 * D + c) * D, xs, B, D, lane, w);
    const float h0 = p.hh[head(p, l, 0, c)];
#pragma unroll
    for (int b = 0; b < kBlockMaxB; ++b) {
        if (b < B && lane == b) {
            const int chain = b * D + c;
            const size_t r = ring(p, n, l) + chain;
            const float q = u[b] * w[b];
            const float cv = fmaf(h0, q, p.ar[r]);
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

// Layer l, step 2: hidden = GELU(m W1).  One wave per hidden unit.
__global__ void __launch_bounds__(256) k_hy_up(Dev p, int rd, int l) {
    extern __shared__ float xs[];                  // [B][D] swizzled
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int B = p.B, D = p.D;
    stage_rows(xs, p.mb, nullptr, B, D);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= 4 * D) return;
    float s[kBlockMaxB];
    row_dot(p.W1t + ((size_t)l * 4 * D + j) * D, xs, B, D, lane, s);
#pragma unroll
    for (int b = 0; b < kBlockMaxB; ++b) {
        if (b < B && lane == b) {
            const float z = s[b];
            p.hb[(size_t)b * 4 * D + j] = 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
        }
    }
}

// Layer l, step 3: z = hidden W2.  One wave per output channel.
__global__ void __launch_bounds__(256) k_hy_down(Dev p, int rd, int l) {
    extern __shared__ float xs[];                  // [B][4D] swizzled
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int B = p.B, D = p.D;
    stage_rows(xs, p.hb, nullptr, B, 4 * D);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= D) return;
    float s[kBlockMaxB];
    row_dot(p.W2t + ((size_t)l * D + c) * 4 * D, xs, B, 4 * D, lane, s);
#pragma unroll
    for (int b = 0; b < kBlockMaxB; ++b)
        if (b < B && lane == b) p.zb[(size_t)b * D + c] = s[b];
}

// After the last layer: a^{M-1} = RMSNorm(z); output, record, next input tanh(a).
__global__ void __launch_bounds__(256) k_hy_out(Dev p, int rd, float *yext) {
    __shared__ float rs[kBlockMaxB];
    const long long n = position_of(p, rd);
    if (n > p.L) return;
    const int B = p.B, D = p.D, BD = B * D;
    row_rms(p.zb, rs, B, D);
    __syncthreads();
    for (int i = threadIdx.x; i < BD; i += blockDim.x) {
        const float a = p.zb[i] * rs[i / D];
        p.ylast[(size_t)(n - 1) * BD + i] = a;
        if (yext) yext[i] = a;
        if (p.reca) p.reca[((size_t)(n - 1) * p.M + (p.M - 1)) * BD + i] = a;
        p.xin[(size_t)((n + 1) & 1) * BD + i] = apply_map(p.fb, a);
    }
}

// dst[c][r] = src[r][c] for a rows x cols matrix of 16-bit values.
__global__ void __launch_bounds__(256) k_transpose16(const unsigned short *src, unsigned short *dst, int rows,
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
