// Device-side state and helpers shared by every kernel of the library.
//
// Data layout in HBM (fp32 unless noted; M layers, B batch rows, D channels,
// L positions, positions 1-based, "row" r = (l*B + b)*D + c, "chain" = b*D + c):
//   filt  [M][D][L]      filter taps h^l[c][k] (spectra, Lazy baseline)
//   hh    [M][HK][D]     filter heads h^l[c][0..HK-1], channel innermost (red
//                        cells and direct gray blocks: coalesced over channels)
//   htap  [M][D][256]    taps 0..255 per (l, c) in runs s = 0..7 of h[s + 8m],
//                        m < 32: one helper lane's taps of a chunk kernel
//   xr    [W][M][B][D]   ring of recent layer inputs x^l_p, slot p mod W
//   ar    [W][M][B][D]   ring of pending sums for positions p in (n, n+W/2]
//   buf   [M][B][D][L]   row-major history: the inputs of every position up to
//                        the last FFT position (copied from the ring in blocks
//                        of G), and the FFT gray blocks' pending sums for later
//                        positions until they are drained into the ring
//                        (activation reuse, Flash Inference "Speicheroptimierung")
//   recx, recy [L][M][B][D]  optional record of every layer input and output
//   Wt, W1t, W2t, zb, mb, hb, reca   Hyena-style block (see fi_block.h)
//   xin   [2][B][D]      next layer-0 input, double-buffered by position parity
//   ylast [L][B][D]      last layer's mixer output per position
//   stamps[2][L+1] (i64) device wall clock at the end of each position; row 1
//                        holds a second sample where a position ends in
//                        several workgroups at once (the reader takes the max)
//   twid  [NT] (float2)  exp(-2 pi i k / NT), generated in fp64 on the host
//   ptw   [NT/2] (float2) per transform size N: W_{2N}^j of real-spectrum item e
//         (pair_slot) at N/2 + e, also fp64 on the host
//   optw  [NT/2] (float2) per half size M: W_{4M}^k of odd-half item e (odd_slot)
//         at M/2 + e
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fi {

constexpr int kLanes = 64;  // lanes of a wave: one chain per lane, so every access is coalesced

// Positions produced so far, in two slots by parity: the kernels of position
// n read slot (n-1)&1 (holding n-1) and the last kernel of position n writes n
// into slot n&1, so no kernel ever reads the slot it may be overwriting.
struct State {
    long long pos[2];
};

struct Dev {
    const float *filt;
    const float *hh;
    const float *htap;   // [M][D][256] chunk helper taps, permuted (k_taps)
    float *buf;
    float *xr;
    float *ar;
    float *recx;
    float *recy;
    float *xin;
    float *ylast;
    State *st;
    long long *stamps;
    const float2 *twid;
    const float2 *ptw;   // pair twiddles: W_{2N}^j of item e at ptw[N/2 + e]
    const float2 *optw;  // odd-half pair twiddles: W_{4M}^k of odd item e at optw[M/2 + e]
    int M, B, D;
    int logNT;
    long long L;
    int HK;    // filter-head taps kept per (l, c)
    int W;     // ring slots (power of two)
    int G;     // copy/drain block between ring and row-major history
    int map;   // 0 tanh, 1 identity, 2 external, 3 Hyena-style block
    int fb;    // 0 tanh, 1 identity
    // Hyena-style block: transposed bf16 weights and per-position activations
    const unsigned short *Wt;   // [M][3D][D]
    const unsigned short *W1t;  // [M][4D][D]
    const unsigned short *W2t;  // [M][D][4D]
    float *zb;                  // [B][D]   down-projection output (before RMSNorm)
    float *mb;                  // [B][D]   gated mixer output
    float *hb;                  // [B][4D]  GELU hidden units
    float *reca;                // [L][M][B][D] optional record of block outputs
};

// Ring entry of (position pos, layer l, chain 0): add the chain index.
__device__ __forceinline__ size_t ring(const Dev &p, long long pos, int l) {
    return ((size_t)(pos & (p.W - 1)) * p.M + l) * (size_t)(p.B * p.D);
}
__device__ __forceinline__ size_t head(const Dev &p, int l, int k, int c) {
    return ((size_t)l * p.HK + k) * p.D + c;
}

__device__ __forceinline__ float apply_map(int kind, float y) { return kind == 0 ? tanhf(y) : y; }

__device__ __forceinline__ size_t act_row(const Dev &p, int l, int b, int c) {
    return ((size_t)((size_t)l * p.B + b) * p.D + c) * (size_t)p.L;
}
__device__ __forceinline__ size_t filt_row(const Dev &p, int l, int c) {
    return ((size_t)l * p.D + c) * (size_t)p.L;
}

// Position of the kernel: slot rd = (n-1)&1 holds n-1 (rd is a launch argument
// fixed when a position's launches are recorded, so graphs can replay them).
__device__ __forceinline__ long long position_of(const Dev &p, int rd) { return p.st->pos[rd] + 1; }

// End of the last kernel of position n: one block publishes n (into the other
// parity slot, which no kernel of this position reads) and stamps the device
// clock.  The next kernel on the stream sees the new value through the kernel
// boundary.  advance 1: the stamp is block 0's end (for a kernel whose blocks
// all run at once, within a block's run time of the kernel's end); advance 2:
// the last block's end, for kernels of many rounds of blocks.
__device__ __forceinline__ void finish_position(const Dev &p, long long n, int advance) {
    if (!advance) return;
    if (advance == 2) {
        // the last workgroup in dispatch order stamps and publishes n once its
        // own threads are done: blocks are dispatched in order, so it ends
        // within one block's run time of the kernel's end
        if (blockIdx.x == gridDim.x - 1 && blockIdx.y == gridDim.y - 1) {
            __syncthreads();
            if (threadIdx.x == 0) {
                p.stamps[n] = (long long)wall_clock64();
                p.st->pos[(n - 1) & 1] = n - 1;
                p.st->pos[n & 1] = n;
            }
        }
        return;
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        p.stamps[n] = (long long)wall_clock64();
        p.st->pos[n & 1] = n;
    }
}

// Copy helper: every thread of the block moves elements tid, tid+bs, ... of a
// strided index space; loads are issued in batches of 16 before any store, so a
// copy costs a few memory round trips instead of one per element.
template <int BATCH = 16, typename Load, typename Store>
__device__ __forceinline__ void batched_copy(int total, int tid, int bs, Load ld, Store st) {
    for (int base = tid; base < total; base += BATCH * bs) {
        float v[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int i = base + k * bs;
            if (i < total) v[k] = ld(i);
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int i = base + k * bs;
            if (i < total) st(i, v[k]);
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
