// Device-side state and helpers shared by every kernel of the library.
//
// Data layout in HBM (fp32 unless noted; M layers, B batch rows, D channels,
// L positions, positions 1-based, slot t = position - 1):
//   filt  [M][D][L]      filter taps h^l[c][k]
//   buf   [M][B][D][L]   activation rows: slot t holds the layer input x^l_{t+1}
//                        once position t+1 is produced, and the pending sum
//                        for position t+1 before that (activation reuse from
//                        Flash Inference's "Speicheroptimierung")
//   rec   [M][B][D][L]   optional record of every mixer output y^l
//   xin   [2][B][D]      next layer-0 input, double-buffered by position parity
//   ylast [L][B][D]      last layer's mixer output per position
//   stamps[L+1] (i64)    device wall clock at the end of each position
//   twid  [NT] (float2)  exp(-2 pi i k / NT), generated in fp64 on the host
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fi {

struct State {
    long long pos;      // positions produced so far
    unsigned done;      // workgroups finished in the current kernel (last-block pattern)
    unsigned pad;
};

struct Dev {
    const float *filt;
    float *buf;
    float *rec;
    float *xin;
    float *ylast;
    State *st;
    long long *stamps;
    const float2 *twid;
    int M, B, D;
    int logNT;
    long long L;
    int map;   // 0 tanh, 1 identity, 2 external
    int fb;    // 0 tanh, 1 identity
};

__device__ __forceinline__ float apply_map(int kind, float y) { return kind == 0 ? tanhf(y) : y; }

__device__ __forceinline__ size_t act_row(const Dev &p, int l, int b, int c) {
    return ((size_t)((size_t)l * p.B + b) * p.D + c) * (size_t)p.L;
}
__device__ __forceinline__ size_t filt_row(const Dev &p, int l, int c) {
    return ((size_t)l * p.D + c) * (size_t)p.L;
}

// End of the last kernel of a position: the last workgroup to finish stamps
// the device clock and publishes the new position.  No memory fence is needed:
// every workgroup read the position when it started, before it counts itself
// done, and the next kernel (same stream) sees the new position and all of
// this kernel's stores through the kernel boundary.
__device__ __forceinline__ void finish_position(const Dev &p, long long n, int advance) {
    if (!advance) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(&p.st->done, 1u);
        if (prev == gridDim.x - 1) {
            p.stamps[n] = (long long)wall_clock64();
            p.st->done = 0;
            p.st->pos = n;
        }
    }
}

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
    return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}

}  // namespace fi
