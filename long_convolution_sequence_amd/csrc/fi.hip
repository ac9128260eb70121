// Host side of the library: context, workspace layout, the relaxed schedule,
// per-block-size path table (device-timed), graph capture and the C-ABI.
//
// Flash Inference (arXiv 2410.12982), summary page, "Kachelung-Strategie",
// "LCSM-Inferenz-Algorithmus", "Schicht-uebergreifende Parallelisierung",
// "Implementierungsdetails" (graphs per token, filter DFT precomputation,
// per-size preconfiguration) and the rebuttal page (per-shape, per-size
// selection of the fastest block implementation by profiling).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <utility>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fi.h"
#include "fi_block.h"
#include "fi_kernels.h"
#include "fi_fft_kernels.h"
#include "fi_dd_kernels.h"
#include "fi_tables.h"

using namespace fi;

namespace {

constexpr int kMaxDirectLog = 7;   // direct gray blocks exist for U <= 128
constexpr int kMinFftLog = 2;      // FFT gray blocks exist for U >= 4
constexpr int kMaxLdsFftLog = 14;  // largest transform held in one workgroup's LDS (128 KB)
constexpr int kMinSubLog = 12;     // smallest sub-block width a split block may use
constexpr int kMaxLayers = 64;
constexpr int kMaxP = 24;
constexpr int kRing = 512;        // ring slots: pending sums reach at most W/2 = 256 ahead
constexpr int kHeadTaps = 256;    // taps h[0..255] serve direct blocks up to U = 128
constexpr int kChunkEv = -1;      // event-pair class of a timed chunk kernel
constexpr int kChunkBlockLog = 4; // a chunk block graph spans 2^4 - 1 chunks

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Launch shape of the transform kernels of 2^logn points (FftShape on the host).
// threads per block of the transform kernels of 2^logn points (FftShape::TPB)
int fft_tpb(int logn) {
    const int tt = logn >= 4 ? (1 << logn) / 16 : 1;
    return tt > 64 ? tt : 64;
}
int fft_per_block(int logn) { return fft_tpb(logn) / (logn >= 4 ? (1 << logn) / 16 : 1); }

int ilog2_exact(int64_t L) {
    if (L < 1 || (L & (L - 1)) != 0) return -1;
    int p = 0;
    while ((int64_t(1) << p) < L) ++p;
    return p;
}

int ctz64(int64_t n) {
    int q = 0;
    while (((n >> q) & 1) == 0) ++q;
    return q;
}

struct Layout {
    size_t filt = 0, hh = 0, htap = 0, pre = 0, buf = 0, xr = 0, ar = 0, recx = 0, recy = 0, twid = 0, xin = 0, ylast = 0,
           stamps = 0, state = 0, scratch = 0, wt = 0, w1t = 0, w2t = 0, zb = 0, mb = 0, hb = 0, reca = 0;
    int HK = 0;
    int pre_stride = 0;              // prefill sums per (b, c): positions of a prompt up to L/2
    size_t spec[kMaxP] = {0};
    size_t spec_pair = 0;            // offset spectra for the deferred two-half class (defer_wide = 2)
    size_t total = 0;
    int logNT = 0;
};

bool fft_exists(int q, int P) { return q >= kMinFftLog && q <= P - 1; }
bool direct_exists(int q) { return q <= kMaxDirectLog; }
// Class vlog + 1 runs its transform as two halves of 2^vlog points in one
// workgroup; wider classes are split into K = U / 2^vlog sub-blocks.
bool is_pair(int q, int vlog) { return q == vlog + 1; }
bool is_sub(int q, int vlog) { return q > vlog + 1; }
int sub_k(int q, int vlog) { return 1 << (q - vlog); }
// float4 entries of class q's spectra per (l, c) row
size_t spec_row_f4(int q, int vlog) {
    return is_sub(q, vlog) ? (size_t)(2 * sub_k(q, vlog) - 1) * ((size_t(1) << vlog) / 2) : (size_t(1) << q) / 2;
}
// Deferral of the two-half class (defer_wide = 2): its block runs as
// kPairSubK sub-blocks of half the one-workgroup width, which needs offset
// spectra of that width (kPairSubK * 2 - 1 per (l, c) row) and exists only
// when that width is one the split kernels take.
constexpr int kPairSubK = 4;
bool pair_defer_exists(int P, int vlog) { return vlog - 1 >= kMinSubLog && vlog + 1 <= P - 1; }
size_t pair_spec_row_f4(int vlog) { return (size_t)(2 * kPairSubK - 1) * ((size_t(1) << (vlog - 1)) / 2); }

// Twiddle tables, fp64 on the host (2 NT float2, NT = 2^logNT): W_NT^k, then
// for every transform size N = 2^logn the pair twiddle W_{2N}^j of each
// real-spectrum item, then the odd-half pair twiddles W_{4N}^k.
std::vector<float2> twiddle_tables(int logNT) {
    const size_t nt = size_t(1) << logNT;
    std::vector<float2> tw(2 * nt, make_float2(1.f, 0.f));
    const double pi = 3.14159265358979323846;
    for (size_t k = 0; k < nt; ++k) {
        const double a = -2.0 * pi * (double)k / (double)nt;
        tw[k] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    for (int logn = 2; logn < logNT; ++logn) {
        const int N = 1 << logn;
        for (int e = 1; e < N / 2; ++e) {
            const double a = -pi * (double)pair_slot(logn, e).j / (double)N;
            tw[nt + N / 2 + e] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
        // odd halves of 2N-point transforms: W_{4N}^k
        for (int e = 0; e < N / 2; ++e) {
            const double a = -pi * (double)odd_slot(logn, e).j / (double)(2 * N);
            tw[nt + nt / 2 + N / 2 + e] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    }
    return tw;
}

bool make_layout(int M, int B, int D, int64_t L, const fi_options &o, Layout &lay) {
    const int P = ilog2_exact(L);
    if (M < 1 || M > kMaxLayers || B < 1 || D < 1 || P < 0 || P > kMaxP) return false;
    const int vlog = o.fft_max_log2;
    if (vlog < kMinSubLog || vlog > kMaxLdsFftLog) return false;
    const bool hyena = o.map == FI_MAP_HYENA;
    if (hyena && (D % 8 != 0 || D > kBlockSpan || B > kBlockMaxB)) return false;
    if ((int64_t)B * D > (int64_t(1) << 24)) return false;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o2 = off;
        off = align_up(off + bytes, 256);
        return o2;
    };
    const size_t rowsMD = (size_t)M * D, rowsMBD = (size_t)M * B * D;
    lay.HK = (int)std::min<int64_t>(kHeadTaps, L);
    lay.filt = take(rowsMD * L * sizeof(float));
    lay.hh = take(rowsMD * lay.HK * sizeof(float));
    lay.htap = take(rowsMD * kChunkTapRow * sizeof(float));
    lay.pre_stride = (int)std::min<int64_t>(L, std::max<int64_t>(L / 2, int64_t(1) << (vlog + 1)));
    lay.pre = take((size_t)B * D * lay.pre_stride * sizeof(float));
    lay.buf = take(rowsMBD * L * sizeof(float));
    lay.xr = take((size_t)kRing * rowsMBD * sizeof(float));
    lay.ar = take((size_t)kRing * rowsMBD * sizeof(float));
    lay.recx = o.record ? take(rowsMBD * L * sizeof(float)) : 0;
    lay.recy = o.record ? take(rowsMBD * L * sizeof(float)) : 0;
    if (hyena) {
        const size_t DD = (size_t)D * D;
        lay.wt = take((size_t)M * 3 * DD * 2);
        lay.w1t = take((size_t)M * 4 * DD * 2);
        lay.w2t = take((size_t)M * 4 * DD * 2);
        lay.zb = take((size_t)B * D * sizeof(float));
        lay.mb = take((size_t)B * D * sizeof(float));
        lay.hb = take((size_t)B * 4 * D * sizeof(float));
        lay.reca = o.record ? take(rowsMBD * L * sizeof(float)) : 0;
    }
    for (int q = 0; q < P; ++q) lay.spec[q] = fft_exists(q, P) ? take(rowsMD * spec_row_f4(q, vlog) * 16) : 0;
    const bool pair_defer = o.defer_wide == 2 && pair_defer_exists(P, vlog);
    lay.spec_pair = pair_defer ? take(rowsMD * pair_spec_row_f4(vlog) * 16) : 0;
    // forward sub-block spectra of the widest split class: [M*B*D][U/2] float4
    // (a deferred two-half block needs [M*B*D][kPairSubK * 2^(vlog-1) / 2], less than any split class)
    const size_t scratch_f4 = is_sub(P - 1, vlog) ? (size_t(1) << (P - 1)) / 2
                              : pair_defer            ? kPairSubK * ((size_t(1) << (vlog - 1)) / 2)
                                                      : 0;
    lay.scratch = scratch_f4 ? take(rowsMBD * scratch_f4 * 16) : 0;
    const int nmax_log = std::min(P - 1, vlog);
    lay.logNT = std::max(2, nmax_log + 1);
    lay.twid = take((size_t(2) << lay.logNT) * sizeof(float2));  // twiddles, pair and odd-pair twiddles
    lay.xin = take((size_t)2 * B * D * sizeof(float));
    lay.ylast = take((size_t)L * B * D * sizeof(float));
    lay.stamps = take((size_t)2 * (L + 1) * sizeof(long long));
    lay.state = take(sizeof(State));
    lay.total = off;
    return true;
}

}  // namespace

struct fi_ctx {
    int M = 0, B = 0, D = 0, P = 0;
    int64_t L = 0;
    fi_options opt{};
    hipStream_t stream = nullptr;
    hipStream_t cap = nullptr;  // private stream used only for graph capture
    // Deferred tails of split gray blocks: output sub-blocks 1..K-1 of a split
    // block at n run on `side` while positions n+1 .. n+V-1 proceed; the
    // stream joins `ev_side` before position side_until = n+V.
    hipStream_t side = nullptr;
    hipEvent_t ev_split = nullptr, ev_side = nullptr;
    int64_t side_until = 0;
    bool own_ws = false;
    char *ws = nullptr;
    Layout lay;
    Dev dev{};
    float4 *spec[kMaxP] = {nullptr};
    float4 *spec_pair = nullptr;     // offset spectra of the deferred two-half class, or NULL
    float4 *scratch = nullptr;
    float *pre = nullptr;            // eager prefill sums [B*D][pre_stride]
    int pre_stride = 0;
    int path[kMaxP] = {0};
    double us_direct[kMaxP], us_fft[kMaxP];
    // chunk-path calibration, per candidate first FFT class g: one chunk of 2^g
    // positions and the class-g FFT block after it (us_chunk), the modeled run
    double us_chunk[kMaxP + 1], us_run[kMaxP + 1];
    int64_t pos = 0;
    int mode = 0;  // 0 fresh, 1 tiled, 2 lazy
    bool poisoned = false;
    std::string err;
    int qd = 0;  // first block-size class computed by FFT (classes below are direct)
    bool weights_set = false;
    hipGraphExec_t gclass[kMaxP + 1] = {nullptr};
    hipGraphExec_t gblock = nullptr;
    int block_log = 0;
    // chunk graphs: gchunk[q] = one chunk and the FFT gray blocks of class q at
    // its end (q = P: the chunk that ends at L, no block); gchunks = the
    // 2^chunk_block_log - 1 chunks of an aligned run of 2^chunk_block_log
    // chunks with their FFT blocks (all but the run's last chunk)
    hipGraphExec_t gchunk[kMaxP + 1] = {nullptr};
    hipGraphExec_t gchunks = nullptr;
    int chunk_block_log = 0;
    // FFT gray-block timing: recorded event pairs not yet read, and the sums
    std::vector<hipEvent_t> ev;
    std::vector<int> ev_class;
    std::vector<int> ev_count;  // 1: the pair counts as one launch of its class
    size_t ev_used = 0;
    double blk_ms[kMaxP] = {0};
    int64_t blk_count[kMaxP] = {0};
    double chunk_ms = 0.0;           // event-timed chunk kernels (time_blocks)
    int64_t chunk_count = 0;
    // Chunked direct positions (maps that act channel by channel): chunks of
    // 2^chunk_log positions, chunk_ch chains per workgroup; -1: not available.
    int chunk_log = -1;
    int chunk_ch = 0;
    // The ring holds no valid pending sums after a chunk: the next per-position
    // launch rebuilds it (cleared, then the FFT sums drained into it).
    bool ring_stale = false;
};

namespace {

fi_status fail(fi_ctx *c, fi_status s, const std::string &msg) {
    if (c && c->err.empty()) c->err = msg;
    if (c && s == FI_EDEVICE) c->poisoned = true;
    return s;
}

#define HIPCK(ctx, call)                                                                     \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail((ctx), FI_EDEVICE,                                                   \
                        std::string(#call) + ": " + hipGetErrorString(e_));                  \
    } while (0)

// ---- kernel dispatch over compile-time block sizes -------------------------

// Layers per block of a direct position: enough blocks to spread the U x U
// products, few enough that the red cells are not recomputed needlessly.
int direct_lg(int M, int U) {
    const int lg = U <= 1 ? M : U == 2 ? 9 : U == 4 ? 3 : U == 8 ? 2 : 1;
    return std::min(M, lg);
}
// U = 1 waits on the red cells, not on staging: a small block suffices
int direct_threads(int U) { return U >= 2 ? kDirectThreads : 256; }
// inputs (U) + taps (2U-1) + pending outputs (U) per layer and lane
size_t direct_lds(int LG, int U) { return U > 0 ? (size_t)LG * (4 * U - 1) * 64 * sizeof(float) : 0; }
size_t ring_lds(int LG, int G) { return (size_t)LG * G * 65 * sizeof(float); }

template <int U, bool CHAIN>
hipError_t launch_direct_u(fi_ctx *c, int rd, hipStream_t s, const float *xext, float *yext, int advance,
                           int rowx) {
    const int LG = direct_lg(c->M, U);
    const dim3 grid((c->B * c->D + 63) / 64, (c->M + LG - 1) / LG);
    hipLaunchKernelGGL((k_direct<U, CHAIN>), grid, dim3(direct_threads(U)), direct_lds(LG, U), s, c->dev, rd, LG,
                       xext, yext, advance, rowx);
    return hipGetLastError();
}

template <int U, bool CHAIN>
hipError_t allow_direct_lds_u(fi_ctx *c) {
    const size_t bytes = std::max<size_t>(direct_lds(direct_lg(c->M, U), U), 1);
    return hipFuncSetAttribute((const void *)k_direct<U, CHAIN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <bool CHAIN>
hipError_t allow_direct_lds(fi_ctx *c) {
    hipError_t e = allow_direct_lds_u<0, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<1, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<2, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<4, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<8, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<16, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<32, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<64, CHAIN>(c);
    if (e == hipSuccess) e = allow_direct_lds_u<128, CHAIN>(c);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)k_red_fft<CHAIN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)ring_lds(1, kRing / 2));
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)k_drain, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)ring_lds(1, kRing / 2));
    return e;
}

// q < 0: red cells only (the last position).  rd = (n-1)&1 for position n.
template <bool CHAIN>
hipError_t launch_direct(fi_ctx *c, int rd, int q, hipStream_t s, const float *xext, float *yext, int advance,
                         int rowx = 0) {
    switch (q) {
        case -1: return launch_direct_u<0, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 0: return launch_direct_u<1, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 1: return launch_direct_u<2, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 2: return launch_direct_u<4, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 3: return launch_direct_u<8, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 4: return launch_direct_u<16, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 5: return launch_direct_u<32, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 6: return launch_direct_u<64, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        case 7: return launch_direct_u<128, CHAIN>(c, rd, s, xext, yext, advance, rowx);
        default: return hipErrorInvalidValue;
    }
}

template <bool CHAIN>
hipError_t launch_red_fft(fi_ctx *c, int rd, hipStream_t s, const float *xext, float *yext) {
    const dim3 grid((c->B * c->D + 63) / 64, c->M);
    hipLaunchKernelGGL((k_red_fft<CHAIN>), grid, dim3(kRingThreads), ring_lds(1, c->dev.G), s, c->dev, rd, 1, xext, yext);
    return hipGetLastError();
}

hipError_t launch_drain(fi_ctx *c, int rd, hipStream_t s, int advance) {
    const dim3 grid((c->B * c->D + 63) / 64, c->M);
    hipLaunchKernelGGL(k_drain, grid, dim3(kRingThreads), (size_t)c->dev.G * 65 * sizeof(float), s, c->dev, rd, advance);
    return hipGetLastError();
}

// ---- chunked direct positions ----------------------------------------------

constexpr int kLdsBytes = 160 * 1024;
// heads [R] float2, slots [G][kChunkSlot], zero rows [kChunkZeroRows][kChunkSlot],
// teacher-forced inputs [G][CH]; R = CH * M
size_t chunk_lds(int CH, int M, int logg) {
    const size_t G = (size_t)1 << logg;
    return (G + kChunkZeroRows) * kChunkSlot * sizeof(float) + (size_t)CH * M * sizeof(float2) +
           G * CH * sizeof(float);
}

// Chains per workgroup: about one workgroup per CU, within the helper rows,
// the LDS and the 64 lanes of wave 0.  0: the stack is too deep for one chain.
int choose_chunk_ch(int M, int BD, int logg, int cus) {
    int ch = std::max(1, (BD + cus - 1) / cus);
    ch = std::min(ch, kChunkMaxRows / M);
    while (ch > 1 && chunk_lds(ch, M, logg) > (size_t)kLdsBytes) --ch;
    return std::min(ch, kLanes);
}

// k_chunk<MT, MODE>: MT = M up to kChunkRegLayers (layers in registers), else
// 0; MODE = kChunkRec (records kept) | kChunkTanh (tanh map and feedback)
ChunkK chunk_kernel(const fi_ctx *c) {
    const int mode = (c->opt.record ? kChunkRec : 0) |
                     (c->opt.map == FI_MAP_TANH && c->opt.feedback == FI_FEEDBACK_TANH ? kChunkTanh : 0);
    return chunk_k(c->M <= kChunkRegLayers ? c->M : 0, mode);
}

// ev0/ev1 (optional) are stamped by the dispatch at the kernel's start and end
hipError_t launch_chunk(fi_ctx *c, int64_t cb, const float *xseq, hipStream_t s, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr) {
    const int CH = c->chunk_ch, BD = c->B * c->D;
    const dim3 grid((unsigned)((BD + CH - 1) / CH)), block(kChunkThreads);
    const size_t lds = chunk_lds(CH, c->M, c->chunk_log);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(chunk_kernel(c), grid, block, lds, s, ev0, ev1, 0, c->dev, (long long)cb,
                              1 << c->chunk_log, CH, xseq);
    else
        hipLaunchKernelGGL(chunk_kernel(c), grid, block, lds, s, c->dev, (long long)cb, 1 << c->chunk_log, CH,
                           xseq);
    return hipGetLastError();
}

hipError_t allow_chunk_lds(fi_ctx *c) {
    return hipFuncSetAttribute((const void *)chunk_kernel(c), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)chunk_lds(c->chunk_ch, c->M, c->chunk_log));
}

// Kernel launch that, given events, has the dispatch itself stamp them at the
// kernel's start and end (exact kernel time, no queueing in between).
template <typename F, typename... Args>
void launch_k(F kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, Args... args) {
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev0, ev1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

hipError_t launch_fft_n(fi_ctx *c, int logn, int rd, hipStream_t s, int advance, hipEvent_t ev0, hipEvent_t ev1) {
    const FftTileK k = fft_tile_k(logn);
    if (!k) return hipErrorInvalidValue;
    const long long tiles = (long long)c->M * c->B * c->D, pb = fft_per_block(logn);
    launch_k(k, dim3((unsigned)((tiles + pb - 1) / pb)), dim3(fft_tpb(logn)), s, ev0, ev1, c->dev, rd,
             (const float4 *)c->spec[logn], advance);
    return hipGetLastError();
}

hipError_t launch_spectrum_n(fi_ctx *c, int logn, hipStream_t s, float4 *dst, long long goff, long long stride) {
    const SpectrumK k = spectrum_k(logn);
    if (!k) return hipErrorInvalidValue;
    const long long rows = (long long)c->M * c->D, pb = fft_per_block(logn);
    hipLaunchKernelGGL(k, dim3((unsigned)((rows + pb - 1) / pb)), dim3(fft_tpb(logn)), 0, s, c->dev, dst, goff,
                       stride);
    return hipGetLastError();
}

// True when the gray block of class q leaves output sub-blocks to the side
// stream: the split classes with defer_wide on, and the two-half class too
// with defer_wide = 2.
bool defers(const fi_ctx *c, int q) {
    const int vlog = c->opt.fft_max_log2;
    if (!c->opt.defer_wide || q >= c->P) return false;
    return is_sub(q, vlog) || (c->opt.defer_wide == 2 && is_pair(q, vlog) && c->spec_pair);
}

// Split class q.  Without `defer`: both kernels on s.  With `defer` (the
// position n known): the forward kernel and output sub-block 0 on s, output
// sub-blocks 1..K-1 on the side stream after the forward kernel, timed by
// dv0/dv1 when given.
// The two-half class runs here too when it is deferred (defer_wide = 2): as
// kPairSubK sub-blocks of half the one-workgroup width, against the offset
// spectra of that width.
hipError_t launch_fft_sub(fi_ctx *c, int rd, int q, hipStream_t s, int advance, hipEvent_t ev0, hipEvent_t ev1,
                          int64_t defer = 0, hipEvent_t dv0 = nullptr, hipEvent_t dv1 = nullptr) {
    const bool pair = is_pair(q, c->opt.fft_max_log2);
    if (pair && !c->spec_pair) return hipErrorInvalidValue;
    const int LOGV = pair ? c->opt.fft_max_log2 - 1 : c->opt.fft_max_log2;
    const int K = pair ? kPairSubK : sub_k(q, LOGV);
    const SubFwdK kf = sub_fwd_k(LOGV);
    const SubInvK ki = sub_inv_k(LOGV, K);
    if (!kf || !ki) return hipErrorInvalidValue;
    const long long rows = (long long)c->M * c->B * c->D;
    const dim3 blk(fft_tpb(LOGV));
    launch_k(kf, dim3((unsigned)(rows * K)), blk, s, ev0, nullptr, c->dev, rd, c->scratch, K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float4 *A = c->scratch, *G = pair ? c->spec_pair : c->spec[q];
    if (!defer) {
        launch_k(ki, dim3((unsigned)(rows * K)), blk, s, nullptr, ev1, c->dev, rd, A, G, K, 0, K, 0LL, advance);
        return hipGetLastError();
    }
    launch_k(ki, dim3((unsigned)rows), blk, s, nullptr, ev1, c->dev, rd, A, G, K, 0, 1, 0LL, advance);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the deferred sub-blocks start once sub-block 0 is done, so they never
    // compete with the position's critical path
    if ((e = hipEventRecord(c->ev_split, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(c->side, c->ev_split, 0)) != hipSuccess) return e;
    launch_k(ki, dim3((unsigned)(rows * (K - 1))), blk, c->side, dv0, dv1, c->dev, rd, A, G, K, 1, K - 1,
             (long long)defer, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(c->ev_side, c->side)) != hipSuccess) return e;
    c->side_until = defer + (int64_t(1) << LOGV);
    return hipSuccess;
}

hipError_t launch_fft2_m(fi_ctx *c, int logm, int rd, hipStream_t s, int advance, hipEvent_t ev0, hipEvent_t ev1) {
    const FftTileK k = fft_tile2_k(logm);
    if (!k) return hipErrorInvalidValue;
    const long long tiles = (long long)c->M * c->B * c->D, pb = fft_per_block(logm);
    launch_k(k, dim3((unsigned)((tiles + pb - 1) / pb)), dim3(fft_tpb(logm)), s, ev0, ev1, c->dev, rd,
             (const float4 *)c->spec[logm + 1], advance);
    return hipGetLastError();
}

// FFT gray blocks of class q; ev0/ev1 (optional) are stamped at the start of
// the first kernel and the end of the last.
hipError_t launch_fft(fi_ctx *c, int rd, int q, hipStream_t s, int advance, hipEvent_t ev0 = nullptr,
                      hipEvent_t ev1 = nullptr) {
    if (is_sub(q, c->opt.fft_max_log2)) return launch_fft_sub(c, rd, q, s, advance, ev0, ev1);
    if (is_pair(q, c->opt.fft_max_log2)) return launch_fft2_m(c, c->opt.fft_max_log2, rd, s, advance, ev0, ev1);
    return launch_fft_n(c, q, rd, s, advance, ev0, ev1);
}

hipError_t launch_spectrum2_m(fi_ctx *c, int logm, hipStream_t s, float4 *dst, long long goff, long long stride) {
    const SpectrumK k = spectrum2_k(logm);
    if (!k) return hipErrorInvalidValue;
    const long long rows = (long long)c->M * c->D, pb = fft_per_block(logm);
    hipLaunchKernelGGL(k, dim3((unsigned)((rows + pb - 1) / pb)), dim3(fft_tpb(logm)), 0, s, c->dev, dst, goff,
                       stride);
    return hipGetLastError();
}

hipError_t launch_spectrum(fi_ctx *c, int q, hipStream_t s) {
    float4 *dst = c->spec[q];
    const int vlog = c->opt.fft_max_log2;
    const long long stride = (long long)spec_row_f4(q, vlog);
    if (is_sub(q, vlog)) {
        // offset spectra d = 1 .. 2K-1: taps h[(d-1)V .. (d+1)V-1]
        const long long V = 1LL << vlog;
        for (int d = 1; d <= 2 * sub_k(q, vlog) - 1; ++d) {
            float4 *dd = dst + (d - 1) * (V / 2);
            const long long goff = (d - 1) * V;
            hipError_t e = launch_spectrum_n(c, vlog, s, dd, goff, stride);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (is_pair(q, vlog)) return launch_spectrum2_m(c, vlog, s, dst, 0, stride);
    return launch_spectrum_n(c, q, s, dst, 0, stride);
}

// All kernels of one position of class q (q == P: the last position, red cells only).
//   direct class:  [red cells + direct gray block]
//   FFT class:     [red cells + ring -> history copy] [FFT gray block] [drain]
// defer > 0 (the position n): a split gray block leaves its later output
// sub-blocks to the side stream.
template <bool CHAIN>
hipError_t launch_position_t(fi_ctx *c, int rd, int q, hipStream_t s, const float *xext, float *yext,
                             int advance, int64_t defer = 0) {
    if (q >= c->P) return launch_direct<CHAIN>(c, rd, -1, s, xext, yext, advance);
    if (q < c->qd) return launch_direct<CHAIN>(c, rd, q, s, xext, yext, advance);
    hipError_t e = launch_red_fft<CHAIN>(c, rd, s, xext, yext);
    if (defer && !c->opt.defer_wide) defer = 0;
    if (e == hipSuccess)
        e = defer && defers(c, q) ? launch_fft_sub(c, rd, q, s, 0, nullptr, nullptr, defer)
                                                    : launch_fft(c, rd, q, s, 0);
    if (e == hipSuccess) e = launch_drain(c, rd, s, advance);
    return e;
}

// Hyena-style block position: per layer projection + red cell, GELU up,
// down; then the output / feedback; then every layer's gray block.
// The block kernels of one position (every layer's projection with its red
// cell, GELU up, down; then the output / feedback).
hipError_t launch_hyena_block(fi_ctx *c, int rd, hipStream_t s, const float *xext, float *yext) {
    const int B = c->B, D = c->D;
    const HyProjK kp = hy_proj_k(B);
    const HyStepK ku = hy_up_k(B), kd = hy_down_k(B);
    if (!kp || !ku || !kd) return hipErrorInvalidValue;
    for (int l = 0; l < c->M; ++l) {
        hipLaunchKernelGGL(kp, dim3((D + 3) / 4), dim3(256), 0, s, c->dev, rd, l, l == 0 ? xext : nullptr);
        hipLaunchKernelGGL(ku, dim3((4 * D / kBlockRows + 3) / 4), dim3(256), 0, s, c->dev, rd, l);
        hipLaunchKernelGGL(kd, dim3((D + kBlockRows - 1) / kBlockRows), dim3(256), 0, s, c->dev, rd, l);
    }
    hipLaunchKernelGGL(k_hy_out, dim3((unsigned)((B * D + 255) / 256)), dim3(256), 0, s, c->dev, rd, yext);
    return hipGetLastError();
}

hipError_t launch_hyena_position(fi_ctx *c, int rd, int q, hipStream_t s, const float *xext, float *yext,
                                 int advance, int64_t defer = 0) {
    hipError_t e = launch_hyena_block(c, rd, s, xext, yext);
    if (e != hipSuccess) return e;
    return launch_position_t<false>(c, rd, q, s, nullptr, nullptr, advance, defer);
}

hipError_t launch_position(fi_ctx *c, int rd, int q, hipStream_t s, const float *xext, float *yext,
                           int advance, int64_t defer = 0) {
    if (c->opt.map == FI_MAP_HYENA) return launch_hyena_position(c, rd, q, s, xext, yext, advance, defer);
    return launch_position_t<true>(c, rd, q, s, xext, yext, advance, defer);
}

// Gray blocks only (external-block mode): the layer inputs at n are in place.
hipError_t launch_tiles(fi_ctx *c, int rd, int q, hipStream_t s, int64_t defer = 0) {
    return launch_position_t<false>(c, rd, q, s, nullptr, nullptr, 1, defer);
}

// Parity slot read by the kernels of position n.
int rd_of(int64_t n) { return (int)((n - 1) & 1); }

int class_of(const fi_ctx *c, int64_t n) { return n < c->L ? ctz64(n) : c->P; }

fi_status check_usable(fi_ctx *c) {
    if (!c) return FI_EINVAL;
    if (c->poisoned) return FI_ESTATE;
    return FI_OK;
}

fi_status set_state_pos(fi_ctx *c, int64_t pos) {
    State st{};
    st.pos[pos & 1] = pos;
    st.pos[(pos & 1) ^ 1] = pos - 1;
    HIPCK(c, hipMemcpyAsync(c->dev.st, &st, sizeof(State), hipMemcpyHostToDevice, c->stream));
    HIPCK(c, hipStreamSynchronize(c->stream));
    return FI_OK;
}

fi_status clear_state(fi_ctx *c) {
    const size_t rowsMBD = (size_t)c->M * c->B * c->D;
    HIPCK(c, hipMemsetAsync(c->dev.buf, 0, rowsMBD * c->L * sizeof(float), c->stream));
    HIPCK(c, hipMemsetAsync(c->dev.xr, 0, (size_t)kRing * rowsMBD * sizeof(float), c->stream));
    HIPCK(c, hipMemsetAsync(c->dev.ar, 0, (size_t)kRing * rowsMBD * sizeof(float), c->stream));
    if (c->dev.recx) {
        HIPCK(c, hipMemsetAsync(c->dev.recx, 0, rowsMBD * c->L * sizeof(float), c->stream));
        HIPCK(c, hipMemsetAsync(c->dev.recy, 0, rowsMBD * c->L * sizeof(float), c->stream));
    }
    if (c->dev.reca) HIPCK(c, hipMemsetAsync(c->dev.reca, 0, rowsMBD * c->L * sizeof(float), c->stream));
    HIPCK(c, hipMemsetAsync(c->dev.xin, 0, 2 * (size_t)c->B * c->D * sizeof(float), c->stream));
    HIPCK(c, hipMemsetAsync(c->dev.ylast, 0, (size_t)c->L * c->B * c->D * sizeof(float), c->stream));
    HIPCK(c, hipMemsetAsync(c->dev.stamps, 0, (size_t)2 * (c->L + 1) * sizeof(long long), c->stream));
    fi_status s = set_state_pos(c, 0);
    if (s != FI_OK) return s;
    c->pos = 0;
    c->mode = 0;
    for (int q = 0; q < kMaxP; ++q) {
        c->blk_ms[q] = 0.0;
        c->blk_count[q] = 0;
    }
    c->ev_used = 0;
    c->ring_stale = false;
    return FI_OK;
}

// Time both gray-block paths of class q at the real shape, n = 2^q, without
// publishing positions.  Protocol: 2 warm-up launches, then the mean of 4
// batches of 8 launches (the pages use 2 warm-ups and the mean of 4 runs).
fi_status time_class(fi_ctx *c, int q, double &us_direct, double &us_fft) {
    us_direct = us_fft = -1.0;
    fi_status st = set_state_pos(c, (int64_t(1) << q) - 1);
    if (st != FI_OK) return st;
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    for (int which = 0; which < 2; ++which) {
        const bool direct = which == 0;
        if (direct && !direct_exists(q)) continue;
        if (!direct && !fft_exists(q, c->P)) continue;
        // the FFT path is timed as if q were the first FFT class (copy/drain block G = U)
        c->dev.G = 1 << q;
        const int rd = rd_of(int64_t(1) << q);
        auto run = [&]() -> hipError_t {
            if (direct) return launch_direct<true>(c, rd, q, c->stream, nullptr, nullptr, 0);
            hipError_t e = launch_red_fft<true>(c, rd, c->stream, nullptr, nullptr);
            if (e == hipSuccess) e = launch_fft(c, rd, q, c->stream, 0);
            if (e == hipSuccess) e = launch_drain(c, rd, c->stream, 0);
            return e;
        };
        for (int w = 0; w < 2; ++w) HIPCK(c, run());
        double total = 0.0;
        for (int rep = 0; rep < 4; ++rep) {
            HIPCK(c, hipEventRecord(a, c->stream));
            for (int k = 0; k < 8; ++k) HIPCK(c, run());
            HIPCK(c, hipEventRecord(b, c->stream));
            HIPCK(c, hipEventSynchronize(b));
            float ms = 0.f;
            HIPCK(c, hipEventElapsedTime(&ms, a, b));
            total += ms * 1000.0 / 8.0;
        }
        (direct ? us_direct : us_fft) = total / 4.0;
    }
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    return FI_OK;
}

// Chunks of 2^g positions for this context: chains per workgroup and the LDS
// attribute.  False when a chunk cannot hold the stack (too deep).
bool setup_chunks(fi_ctx *c, int g, int cus) {
    c->chunk_log = g;
    c->chunk_ch = choose_chunk_ch(c->M, c->B * c->D, g, cus);
    if (c->chunk_ch < 1) {
        c->chunk_log = -1;
        return false;
    }
    return allow_chunk_lds(c) == hipSuccess;
}

// Mean microseconds of the FFT gray-block kernels of class q alone, at n = 2^q
// (2 warm-up launches, then 4 batches of 8).
fi_status time_fft_only(fi_ctx *c, int q, double &us) {
    us = -1.0;
    fi_status st = set_state_pos(c, (int64_t(1) << q) - 1);
    if (st != FI_OK) return st;
    const int rd = rd_of(int64_t(1) << q);
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    for (int w = 0; w < 2; ++w) HIPCK(c, launch_fft(c, rd, q, c->stream, 0));
    double total = 0.0;
    for (int rep = 0; rep < 4; ++rep) {
        HIPCK(c, hipEventRecord(a, c->stream));
        for (int k = 0; k < 8; ++k) HIPCK(c, launch_fft(c, rd, q, c->stream, 0));
        HIPCK(c, hipEventRecord(b, c->stream));
        HIPCK(c, hipEventSynchronize(b));
        float ms = 0.f;
        HIPCK(c, hipEventElapsedTime(&ms, a, b));
        total += ms * 1000.0 / 8.0;
    }
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    us = total / 4.0;
    return FI_OK;
}

// Mean microseconds of one chunk of the first G = 2^chunk_log positions, then
// the FFT gray blocks of class chunk_log at its end (none when the chunk ends
// at L): launched back to back as in a generation, one warm-up and three timed
// pairs, the chunk's pending sums cleared before each.
fi_status time_chunk_pair(fi_ctx *c, double &us) {
    us = -1.0;
    const int g = c->chunk_log;
    const int64_t G = int64_t(1) << g;
    const size_t rows = (size_t)c->M * c->B * c->D;
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    double total = 0.0;
    for (int rep = 0; rep < 4; ++rep) {
        fi_status st = set_state_pos(c, 0);
        if (st != FI_OK) return st;
        HIPCK(c, hipMemset2DAsync(c->dev.buf, (size_t)c->L * sizeof(float), 0, (size_t)G * sizeof(float), rows,
                                  c->stream));
        HIPCK(c, hipEventRecord(a, c->stream));
        HIPCK(c, launch_chunk(c, 0, nullptr, c->stream));
        if (g < c->P) HIPCK(c, launch_fft(c, rd_of(G), g, c->stream, 2));
        HIPCK(c, hipEventRecord(b, c->stream));
        HIPCK(c, hipEventSynchronize(b));
        float ms = 0.f;
        HIPCK(c, hipEventElapsedTime(&ms, a, b));
        if (rep > 0) total += ms * 1000.0;
    }
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    us = total / 3.0;
    return FI_OK;
}

// The hybrid split for chunked positions, timed on the path it configures
// (rebuttal page: profile per shape and block size, pick the fastest): for
// each candidate first FFT class g, a chunk of 2^g positions carries every
// block below 2^g, and classes from g on run as FFT blocks.  The whole run
// costs (L / 2^g) chunks plus 2^(P-1-q) FFT blocks of each class q >= g; the
// classes above kMaxDirectLog + 1 are FFT blocks for every candidate and are
// left out of the comparison.  Picks into qd the least g whose modeled run is
// within kSplitTie of the cheapest: one chunk pair is timed to about 1%, and
// candidates that close (chunks of 128 and 256 on the 18 x 864 x 2^17 stack,
// 0.2-1% apart either way from one calibration to the next) would otherwise
// be chosen by noise.  Of two such, the shorter chunk runs every position at
// the red-cell chain's pace; the longer has positions bound by its helpers,
// which one timed pair weighs less than whole generations do (there the
// shorter was 0.4-0.6% faster).
constexpr double kSplitTie = 0.015;
fi_status calibrate_chunks(fi_ctx *c, int cus, int &qd) {
    const int qtop = std::min(kMaxDirectLog + 1, c->P - 1);      // FFT classes that may switch
    for (int q = kMinFftLog; q <= qtop; ++q) {
        fi_status st = time_fft_only(c, q, c->us_fft[q]);
        if (st != FI_OK) return st;
    }
    double best = -1.0;
    for (int g = kMinFftLog; g <= std::min(kMaxDirectLog + 1, c->P); ++g) {
        if (!setup_chunks(c, g, cus)) continue;
        fi_status st = time_chunk_pair(c, c->us_chunk[g]);
        if (st != FI_OK) return st;
        double cost = std::ldexp(c->us_chunk[g] - (g < c->P ? c->us_fft[g] : 0.0), c->P - g);
        for (int q = g; q <= qtop; ++q) cost += std::ldexp(c->us_fft[q], c->P - 1 - q);
        c->us_run[g] = cost;
        if (best < 0 || cost < best) best = cost;
    }
    for (int g = kMinFftLog; g <= std::min(kMaxDirectLog + 1, c->P); ++g)
        if (c->us_run[g] >= 0 && c->us_run[g] <= best * (1.0 + kSplitTie)) {
            qd = g;
            break;
        }
    return clear_state(c);
}

// Record the positions (class, parity slot) into one graph.
fi_status capture(fi_ctx *c, hipGraphExec_t *out, const std::vector<std::pair<int, int>> &positions) {
    hipGraph_t g = nullptr;
    HIPCK(c, hipStreamBeginCapture(c->cap, hipStreamCaptureModeThreadLocal));
    hipError_t err = hipSuccess;
    for (const auto &qr : positions) {
        err = launch_position(c, qr.second, qr.first, c->cap, nullptr, nullptr, 1);
        if (err != hipSuccess) break;
    }
    hipError_t e2 = hipStreamEndCapture(c->cap, &g);
    if (err != hipSuccess) return fail(c, FI_EDEVICE, std::string("capture: ") + hipGetErrorString(err));
    if (e2 != hipSuccess) return fail(c, FI_EDEVICE, std::string("end capture: ") + hipGetErrorString(e2));
    hipError_t e3 = hipGraphInstantiate(out, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e3 != hipSuccess) return fail(c, FI_EDEVICE, std::string("instantiate: ") + hipGetErrorString(e3));
    return FI_OK;
}

// Record chunk launches into one graph: for each entry, a chunk (its base read
// from the published position) and, for q < P, the FFT gray blocks of class q
// at its end.
fi_status capture_chunks(fi_ctx *c, hipGraphExec_t *out, const std::vector<int> &classes) {
    hipGraph_t g = nullptr;
    HIPCK(c, hipStreamBeginCapture(c->cap, hipStreamCaptureModeThreadLocal));
    hipError_t err = hipSuccess;
    for (int q : classes) {
        err = launch_chunk(c, -1, nullptr, c->cap);
        if (err == hipSuccess && q < c->P) err = launch_fft(c, 1, q, c->cap, 2);
        if (err != hipSuccess) break;
    }
    hipError_t e2 = hipStreamEndCapture(c->cap, &g);
    if (err != hipSuccess) return fail(c, FI_EDEVICE, std::string("capture: ") + hipGetErrorString(err));
    if (e2 != hipSuccess) return fail(c, FI_EDEVICE, std::string("end capture: ") + hipGetErrorString(e2));
    hipError_t e3 = hipGraphInstantiate(out, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e3 != hipSuccess) return fail(c, FI_EDEVICE, std::string("instantiate: ") + hipGetErrorString(e3));
    return FI_OK;
}

fi_status build_graphs(fi_ctx *c) {
    // class q: n odd iff q == 0; the last position L is even
    for (int q = 0; q <= c->P; ++q) {
        fi_status s = capture(c, &c->gclass[q], {{q, q == 0 ? 0 : 1}});
        if (s != FI_OK) return s;
    }
    // positions m*2^k + j, j = 1 .. 2^k-1: class ctz(j), parity of j
    // (a block-mode position is ~3M+5 kernels: only the per-class graphs there)
    const int k = c->opt.map == FI_MAP_HYENA ? 0 : c->opt.block_graph_log2;
    if (k >= 1 && k < c->P) {
        std::vector<std::pair<int, int>> pos;
        for (int64_t j = 1; j < (int64_t(1) << k); ++j) pos.push_back({ctz64(j), rd_of(j)});
        fi_status s = capture(c, &c->gblock, pos);
        if (s != FI_OK) return s;
        c->block_log = k;
    }
    if (c->chunk_log >= 0) {
        // chunk q_end = class of the position that ends it; chunks end at
        // multiples of G = 2^chunk_log, so q_end >= chunk_log
        for (int q = c->chunk_log; q <= c->P; ++q) {
            fi_status s = capture_chunks(c, &c->gchunk[q], {q});
            if (s != FI_OK) return s;
        }
        const int kb = std::min(kChunkBlockLog, c->P - c->chunk_log - 1);
        if (kb >= 1) {
            std::vector<int> classes;
            for (int j = 1; j < (1 << kb); ++j) classes.push_back(c->chunk_log + ctz64(j));
            fi_status s = capture_chunks(c, &c->gchunks, classes);
            if (s != FI_OK) return s;
            c->chunk_block_log = kb;
        }
    }
    return FI_OK;
}

void destroy_graphs(fi_ctx *c) {
    for (auto &g : c->gclass)
        if (g) {
            (void)hipGraphExecDestroy(g);
            g = nullptr;
        }
    if (c->gblock) (void)hipGraphExecDestroy(c->gblock);
    c->gblock = nullptr;
    for (auto &g : c->gchunk)
        if (g) {
            (void)hipGraphExecDestroy(g);
            g = nullptr;
        }
    if (c->gchunks) (void)hipGraphExecDestroy(c->gchunks);
    c->gchunks = nullptr;
    for (auto &e : c->ev)
        if (e) (void)hipEventDestroy(e);
    c->ev.clear();
}

// Read every recorded event pair into the per-class sums (synchronises).
fi_status harvest_events(fi_ctx *c) {
    if (c->ev_used == 0) return FI_OK;
    HIPCK(c, hipStreamSynchronize(c->stream));
    HIPCK(c, hipStreamSynchronize(c->side));
    for (size_t i = 0; i < c->ev_used; ++i) {
        float ms = 0.f;
        HIPCK(c, hipEventElapsedTime(&ms, c->ev[2 * i], c->ev[2 * i + 1]));
        if (c->ev_class[i] == kChunkEv) {
            c->chunk_ms += ms;
            c->chunk_count += c->ev_count[i];
        } else {
            c->blk_ms[c->ev_class[i]] += ms;
            c->blk_count[c->ev_class[i]] += c->ev_count[i];
        }
    }
    c->ev_used = 0;
    return FI_OK;
}

// Room for two more event pairs (harvesting the pool when it is full).
fi_status reserve_events(fi_ctx *c) {
    constexpr size_t kPairs = 4096;
    if (c->ev.empty()) {
        c->ev.resize(2 * kPairs, nullptr);
        c->ev_class.resize(kPairs, 0);
        c->ev_count.resize(kPairs, 0);
        for (auto &e : c->ev) HIPCK(c, hipEventCreate(&e));
    }
    if (c->ev_used + 2 > kPairs) return harvest_events(c);
    return FI_OK;
}

// The FFT gray blocks of position n (class q), timed by events that their
// dispatch stamps.
fi_status launch_timed_fft(fi_ctx *c, int64_t n, int q, int advance) {
    const int rd = rd_of(n);
    fi_status s0 = reserve_events(c);
    if (s0 != FI_OK) return s0;
    const size_t i = c->ev_used++;
    c->ev_class[i] = q;
    c->ev_count[i] = 1;
    if (defers(c, q)) {
        // the deferred sub-blocks' kernel time adds to this launch
        const size_t j = c->ev_used++;
        c->ev_class[j] = q;
        c->ev_count[j] = 0;
        HIPCK(c, launch_fft_sub(c, rd, q, c->stream, advance, c->ev[2 * i], c->ev[2 * i + 1], n, c->ev[2 * j],
                                c->ev[2 * j + 1]));
    } else {
        HIPCK(c, launch_fft(c, rd, q, c->stream, advance, c->ev[2 * i], c->ev[2 * i + 1]));
    }
    return FI_OK;
}

// One FFT-class position launched directly, its gray-block kernels timed.
fi_status launch_timed_position(fi_ctx *c, int64_t n, int q) {
    const int rd = rd_of(n);
    HIPCK(c, launch_red_fft<true>(c, rd, c->stream, nullptr, nullptr));
    fi_status s = launch_timed_fft(c, n, q, 0);
    if (s != FI_OK) return s;
    HIPCK(c, launch_drain(c, rd, c->stream, 1));
    return FI_OK;
}

// Positions cb+1 .. cb+G as one chunk launch, then the FFT gray blocks of
// position cb+G (none at L).  xseq: teacher-forced inputs [G][B][D] or NULL.
fi_status run_chunk(fi_ctx *c, int64_t cb, const float *xseq) {
    const int64_t n = cb + (int64_t(1) << c->chunk_log);
    if (c->opt.time_blocks) {
        fi_status s = reserve_events(c);
        if (s != FI_OK) return s;
        const size_t i = c->ev_used++;
        c->ev_class[i] = kChunkEv;
        c->ev_count[i] = 1;
        HIPCK(c, launch_chunk(c, cb, xseq, c->stream, c->ev[2 * i], c->ev[2 * i + 1]));
    } else {
        HIPCK(c, launch_chunk(c, cb, xseq, c->stream));
    }
    c->ring_stale = true;
    if (n >= c->L) return FI_OK;
    const int q = class_of(c, n);
    // the gray block's last kernel is stamped and published by its last
    // workgroup (for the widest blocks block 0 ends far earlier)
    if (c->opt.time_blocks) {
        fi_status s = launch_timed_fft(c, n, q, 2);
        if (s != FI_OK) return s;
    } else if (defers(c, q)) {
        HIPCK(c, launch_fft_sub(c, rd_of(n), q, c->stream, 2, nullptr, nullptr, n));
    } else {
        HIPCK(c, launch_fft(c, rd_of(n), q, c->stream, 2));
    }
    return FI_OK;
}

// True when the positions pos+1 .. pos+G form a whole chunk inside the run.
bool chunk_fits(const fi_ctx *c, int64_t pos, int64_t end) {
    if (c->chunk_log < 0 || !c->opt.chunk_direct) return false;
    const int64_t G = int64_t(1) << c->chunk_log;
    return (pos & (G - 1)) == 0 && pos + G <= end;
}

// Before a per-position launch after chunks: clear the ring's pending sums and
// drain the FFT sums of the next G positions into it (the chunk kernel kept
// them in the row-major history only).  Direct gray blocks never cross a
// multiple of G, so nothing else is pending there.
fi_status resume_ring(fi_ctx *c) {
    if (!c->ring_stale) return FI_OK;
    const size_t rows = (size_t)c->M * c->B * c->D;
    HIPCK(c, hipMemsetAsync(c->dev.ar, 0, (size_t)kRing * rows * sizeof(float), c->stream));
    const int64_t G = c->dev.G;
    if (G && c->pos > 0 && c->pos % G == 0 && c->pos + G <= c->L)
        HIPCK(c, launch_drain(c, rd_of(c->pos), c->stream, 0));
    c->ring_stale = false;
    return FI_OK;
}

// Before launching positions up to `upto` (the last position whose kernels,
// its gray block included, the launch issues: for a chunk of positions
// pos+1 .. pos+G that is pos+G, whose FFT block run_chunk launches too): join
// the side stream if deferred sub-blocks it still computes are due by then
// (upto < 0: join in any case).  The block of position side_until writes into
// the first deferred sub-block, so it must not start before the side stream
// is done.
fi_status join_side(fi_ctx *c, int64_t upto) {
    if (c->side_until && (upto < 0 || upto >= c->side_until)) {
        HIPCK(c, hipStreamWaitEvent(c->stream, c->ev_side, 0));
        c->side_until = 0;
    }
    return FI_OK;
}

// The kernels of one baseline position n (rd its parity slot).  Lazy: the
// full sum of every row, then the red cells.  Eager: the red cells, then every
// row's push into the later pending sums.  _NP: the per-row work launched
// layer by layer instead of for all layers at once ([S] "Vergleichsmethoden",
// Lazy NP / Eager NP).  advance = 0 leaves the position unpublished (timing).
hipError_t launch_baseline(fi_ctx *c, int kind, int rd, int64_t n, const float *x_t, float *y_t, int advance) {
    const long long BD = (long long)c->B * c->D, rows = BD * c->M;
    const bool np = kind == FI_BASE_LAZY_NP || kind == FI_BASE_EAGER_NP;
    const int parts = np ? c->M : 1;
    const long long per = np ? BD : rows;
    hipError_t e;
    if (kind == FI_BASE_LAZY || kind == FI_BASE_LAZY_NP) {
        for (int k = 0; k < parts; ++k) {
            hipLaunchKernelGGL(k_lazy_dot, dim3((unsigned)per), dim3(256), 0, c->stream, c->dev, rd, k * per);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // red cells; the inputs also go to the row-major history the next sums read
        return launch_direct<true>(c, rd, -1, c->stream, x_t, y_t, advance, 1);
    }
    if ((e = launch_direct<true>(c, rd, -1, c->stream, x_t, y_t, advance, 1)) != hipSuccess) return e;
    if (n >= c->L) return hipSuccess;
    const unsigned spans = (unsigned)((c->L - n + kEagerSpan - 1) / kEagerSpan);
    for (int k = 0; k < parts; ++k) {
        hipLaunchKernelGGL(k_eager_push, dim3(spans, (unsigned)per), dim3(256), 0, c->stream, c->dev, rd, k * per);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

fi_status enter_mode(fi_ctx *c, int mode) {
    if (c->mode != 0 && c->mode != mode)
        return fail(c, FI_ESTATE, "tiled, Lazy and Eager calls cannot be mixed without fi_reset");
    c->mode = mode;
    return FI_OK;
}

}  // namespace

extern "C" {

void fi_default_options(fi_options *o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->map = FI_MAP_TANH;
    o->feedback = FI_FEEDBACK_TANH;
    o->tau_mode = FI_TAU_AUTO;
    o->tau_split = -1;
    o->record = 0;
    o->use_graphs = 1;
    o->block_graph_log2 = 6;
    o->filters_on_device = 0;
    o->fft_max_log2 = kMaxLdsFftLog;
    o->chunk_direct = 1;
    o->eager_prefill = 1;
}

const char *fi_version(void) { return "fi 0.1 gfx950"; }

size_t fi_workspace_bytes(int layers, int batch, int channels, int64_t L, const fi_options *opt) {
    fi_options o;
    if (opt)
        o = *opt;
    else
        fi_default_options(&o);
    Layout lay;
    if (!make_layout(layers, batch, channels, L, o, lay)) return 0;
    return lay.total;
}

fi_status fi_init(fi_ctx **out, int layers, int batch, int channels, int64_t L, const float *filters,
                  const fi_options *opt, void *workspace, void *stream) {
    if (!out) return FI_EINVAL;
    *out = nullptr;
    if (!filters) return FI_EINVAL;
    fi_options o;
    if (opt)
        o = *opt;
    else
        fi_default_options(&o);
    if (o.map < FI_MAP_TANH || o.map > FI_MAP_HYENA) return FI_EINVAL;
    if (o.feedback < FI_FEEDBACK_TANH || o.feedback > FI_FEEDBACK_IDENTITY) return FI_EINVAL;
    if (o.defer_wide < 0 || o.defer_wide > 2) return FI_EINVAL;
    if (o.chunk_direct != 0 && o.chunk_direct != 1) return FI_EINVAL;
    for (int r : o.reserved)
        if (r != 0) return FI_EINVAL;
    if (o.tau_mode < FI_TAU_AUTO || o.tau_mode > FI_TAU_FFT) return FI_EINVAL;
    if ((uintptr_t)workspace % 256 != 0) return FI_EINVAL;
    Layout lay;
    if (!make_layout(layers, batch, channels, L, o, lay)) return FI_EINVAL;

    fi_ctx *c = new fi_ctx();
    c->M = layers;
    c->B = batch;
    c->D = channels;
    c->L = L;
    c->P = ilog2_exact(L);
    c->opt = o;
    c->lay = lay;
    c->stream = (hipStream_t)stream;
    for (int q = 0; q < kMaxP; ++q) c->us_direct[q] = c->us_fft[q] = -1.0;
    for (int q = 0; q <= kMaxP; ++q) c->us_chunk[q] = c->us_run[q] = -1.0;

    auto bail = [&](fi_status s) {
        fi_destroy(c);
        return s;
    };
    if (workspace) {
        c->ws = (char *)workspace;
    } else {
        if (hipMalloc((void **)&c->ws, lay.total) != hipSuccess) {
            (void)hipGetLastError();
            c->ws = nullptr;
            return bail(FI_ENOMEM);
        }
        c->own_ws = true;
    }
    if (hipStreamCreateWithFlags(&c->cap, hipStreamNonBlocking) != hipSuccess) return bail(FI_EDEVICE);
    if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_split, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->ev_side, hipEventDisableTiming) != hipSuccess)
        return bail(FI_EDEVICE);

    Dev &d = c->dev;
    d.filt = (const float *)(c->ws + lay.filt);
    d.hh = (const float *)(c->ws + lay.hh);
    d.htap = (const float *)(c->ws + lay.htap);
    d.buf = (float *)(c->ws + lay.buf);
    d.xr = (float *)(c->ws + lay.xr);
    d.ar = (float *)(c->ws + lay.ar);
    d.recx = o.record ? (float *)(c->ws + lay.recx) : nullptr;
    d.recy = o.record ? (float *)(c->ws + lay.recy) : nullptr;
    d.HK = lay.HK;
    d.W = kRing;
    d.G = 0;
    d.xin = (float *)(c->ws + lay.xin);
    d.ylast = (float *)(c->ws + lay.ylast);
    d.st = (State *)(c->ws + lay.state);
    d.stamps = (long long *)(c->ws + lay.stamps);
    d.twid = (const float2 *)(c->ws + lay.twid);
    d.ptw = d.twid + (size_t(1) << lay.logNT);
    d.optw = d.ptw + (size_t(1) << (lay.logNT - 1));
    d.M = layers;
    d.B = batch;
    d.D = channels;
    d.L = L;
    d.logNT = lay.logNT;
    d.map = o.map == FI_MAP_IDENTITY ? 1 : o.map == FI_MAP_EXTERNAL ? 2 : o.map == FI_MAP_HYENA ? 3 : 0;
    if (o.map == FI_MAP_HYENA) {
        d.Wt = (const unsigned short *)(c->ws + lay.wt);
        d.W1t = (const unsigned short *)(c->ws + lay.w1t);
        d.W2t = (const unsigned short *)(c->ws + lay.w2t);
        d.zb = (float *)(c->ws + lay.zb);
        d.mb = (float *)(c->ws + lay.mb);
        d.hb = (float *)(c->ws + lay.hb);
        d.reca = o.record ? (float *)(c->ws + lay.reca) : nullptr;

    }
    d.fb = o.feedback == FI_FEEDBACK_IDENTITY ? 1 : 0;
    for (int q = 0; q < c->P; ++q)
        c->spec[q] = fft_exists(q, c->P) ? (float4 *)(c->ws + lay.spec[q]) : nullptr;
    c->spec_pair = lay.spec_pair ? (float4 *)(c->ws + lay.spec_pair) : nullptr;
    c->scratch = lay.scratch ? (float4 *)(c->ws + lay.scratch) : nullptr;
    c->pre = (float *)(c->ws + lay.pre);
    c->pre_stride = lay.pre_stride;

    // filters
    const size_t fbytes = (size_t)layers * channels * L * sizeof(float);
    if (hipMemcpyAsync((void *)d.filt, filters, fbytes,
                       o.filters_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                       c->stream) != hipSuccess)
        return bail(fail(c, FI_EDEVICE, "filter copy failed"));
    {
        const std::vector<float2> tw = twiddle_tables(lay.logNT);
        if (hipMemcpyAsync((void *)d.twid, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice,
                           c->stream) != hipSuccess ||
            hipStreamSynchronize(c->stream) != hipSuccess)
            return bail(fail(c, FI_EDEVICE, "twiddle copy failed"));
    }
    // the direct and ring-copy kernels size their LDS at launch (up to 98 KB)
    if (allow_direct_lds<true>(c) != hipSuccess || allow_direct_lds<false>(c) != hipSuccess)
        return bail(fail(c, FI_EDEVICE, "direct kernel LDS attribute"));
    {
        const size_t nh = (size_t)layers * lay.HK * channels;
        hipLaunchKernelGGL(k_heads, dim3((unsigned)((nh + 255) / 256)), dim3(256), 0, c->stream, c->dev,
                           (float *)(c->ws + lay.hh));
        if (hipGetLastError() != hipSuccess) return bail(fail(c, FI_EDEVICE, "filter heads"));
        const size_t nt = (size_t)layers * channels * kChunkTapRow;
        hipLaunchKernelGGL(k_taps, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, c->stream, c->dev,
                           (float *)(c->ws + lay.htap));
        if (hipGetLastError() != hipSuccess) return bail(fail(c, FI_EDEVICE, "chunk tap table"));
    }
    if (clear_state(c) != FI_OK) return bail(FI_EDEVICE);

    // spectra of every class an FFT block may serve
    for (int q = 0; q < c->P; ++q) {
        if (!c->spec[q]) continue;
        if (launch_spectrum(c, q, c->stream) != hipSuccess) return bail(fail(c, FI_EDEVICE, "spectrum launch"));
    }
    if (c->spec_pair) {
        // offset spectra d = 1 .. 2 kPairSubK - 1 of width V = 2^(vlog-1): taps h[(d-1)V .. (d+1)V-1]
        const int plog = o.fft_max_log2 - 1;
        const long long V = 1LL << plog, stride = (long long)pair_spec_row_f4(o.fft_max_log2);
        for (int d = 1; d <= 2 * kPairSubK - 1; ++d)
            if (launch_spectrum_n(c, plog, c->stream, c->spec_pair + (d - 1) * (V / 2), (d - 1) * V, stride) !=
                hipSuccess)
                return bail(fail(c, FI_EDEVICE, "spectrum launch"));
    }

    // Path table.  Blocks of edge 2^q with q < qd are direct, the rest FFT (direct
    // blocks exist up to U = 128, so qd <= 8; FFT blocks from U = 4).  A single
    // split keeps every FFT position a multiple of G = 2^qd, the ring-copy block.
    int qd = std::min(c->P, kMaxDirectLog + 1);              // default: direct wherever it exists
    if (o.tau_mode == FI_TAU_FFT) qd = std::min(c->P, kMinFftLog);
    else if (o.tau_mode == FI_TAU_AUTO && o.tau_split >= 0)
        qd = std::min(c->P, std::max(kMinFftLog, std::min(o.tau_split, kMaxDirectLog + 1)));
    int cus = 0;
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return bail(fail(c, FI_EDEVICE, "device query"));
    }
    const bool chunked = (o.map == FI_MAP_TANH || o.map == FI_MAP_IDENTITY) && o.chunk_direct &&
                         choose_chunk_ch(c->M, c->B * c->D, 0, cus) >= 1;
    if (o.tau_mode == FI_TAU_AUTO && o.tau_split < 0 && chunked) {
        // chunked positions: time the chunk path itself per candidate split
        if (calibrate_chunks(c, cus, qd) != FI_OK) return bail(FI_EDEVICE);
    } else if (o.tau_mode == FI_TAU_AUTO && o.tau_split < 0) {
        // one launch per position: time both paths per class at the real shape,
        // then pick the split that minimises the whole run: class q runs
        // 2^(P-1-q) times
        for (int q = kMinFftLog; q <= std::min(kMaxDirectLog, c->P - 1); ++q) {
            double ud, uf;
            if (time_class(c, q, ud, uf) != FI_OK) return bail(FI_EDEVICE);
            c->us_direct[q] = ud;
            c->us_fft[q] = uf;
        }
        double best = -1.0;
        for (int cand = kMinFftLog; cand <= std::min(kMaxDirectLog + 1, c->P); ++cand) {
            double cost = 0.0;
            for (int q = kMinFftLog; q <= std::min(kMaxDirectLog, c->P - 1); ++q)
                cost += std::ldexp(q < cand ? c->us_direct[q] : c->us_fft[q], c->P - 1 - q);
            if (best < 0 || cost < best) {
                best = cost;
                qd = cand;
            }
        }
        if (clear_state(c) != FI_OK) return bail(FI_EDEVICE);
    }
    c->qd = qd;
    for (int q = 0; q < c->P; ++q) c->path[q] = q < qd ? FI_PATH_DIRECT : FI_PATH_FFT;
    c->dev.G = qd < c->P ? (1 << qd) : 0;
    c->chunk_log = -1;
    if (o.map == FI_MAP_TANH || o.map == FI_MAP_IDENTITY) {
        // chunks end at the FFT positions (or at L when every class is direct);
        // none when the stack is deeper than the helper rows of one workgroup
        if (!setup_chunks(c, std::min(qd, c->P), cus) && c->chunk_log >= 0)
            return bail(fail(c, FI_EDEVICE, "chunk kernel LDS attribute"));
    }
    if (o.use_graphs && o.map != FI_MAP_EXTERNAL) {
        if (build_graphs(c) != FI_OK) return bail(FI_EDEVICE);
    }
    if (hipStreamSynchronize(c->stream) != hipSuccess) return bail(fail(c, FI_EDEVICE, "init sync"));
    *out = c;
    return FI_OK;
}

fi_status fi_destroy(fi_ctx *c) {
    if (!c) return FI_OK;
    if (c->ws) (void)hipStreamSynchronize(c->stream);
    if (c->side) (void)hipStreamSynchronize(c->side);
    destroy_graphs(c);
    if (c->cap) (void)hipStreamDestroy(c->cap);
    if (c->side) (void)hipStreamDestroy(c->side);
    if (c->ev_split) (void)hipEventDestroy(c->ev_split);
    if (c->ev_side) (void)hipEventDestroy(c->ev_side);
    if (c->own_ws && c->ws) (void)hipFree(c->ws);
    delete c;
    return FI_OK;
}

fi_status fi_reset(fi_ctx *c) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = join_side(c, -1)) != FI_OK) return s;
    return clear_state(c);
}

fi_status fi_set_defer_wide(fi_ctx *c, int on) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (on < 0 || on > 2) return FI_EINVAL;
    if (on == 2 && !c->spec_pair && pair_defer_exists(c->P, c->opt.fft_max_log2))
        return fail(c, FI_ESTATE, "defer_wide = 2 needs fi_options.defer_wide = 2 at fi_init (its spectra)");
    if ((s = join_side(c, -1)) != FI_OK) return s;
    c->opt.defer_wide = on;
    return FI_OK;
}

int64_t fi_position(const fi_ctx *c) { return c ? c->pos : -1; }

const char *fi_last_error(const fi_ctx *c) { return c ? c->err.c_str() : "null context"; }

fi_status fi_set_input(fi_ctx *c, const float *x0) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (!x0) return FI_EINVAL;
    // position n reads xin[n & 1]; the next position is pos + 1
    float *dst = c->dev.xin + (size_t)((c->pos + 1) & 1) * c->B * c->D;
    HIPCK(c, hipMemcpyAsync(dst, x0, (size_t)c->B * c->D * sizeof(float), hipMemcpyDeviceToDevice,
                            c->stream));
    return FI_OK;
}

fi_status fi_step(fi_ctx *c, const float *x_t, float *y_t) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map == FI_MAP_EXTERNAL) return fail(c, FI_ESTATE, "fi_step in external-block mode");
    if (c->opt.map == FI_MAP_HYENA && !c->weights_set) return fail(c, FI_ESTATE, "block weights not set");
    if (c->pos >= c->L) return FI_ERANGE;
    if ((s = enter_mode(c, 1)) != FI_OK) return s;
    const int64_t n = c->pos + 1;
    if ((s = join_side(c, n)) != FI_OK) return s;
    if ((s = resume_ring(c)) != FI_OK) return s;
    HIPCK(c, launch_position(c, rd_of(n), class_of(c, n), c->stream, x_t, y_t, 1, n));
    c->pos = n;
    return FI_OK;
}

}  // extern "C"

namespace {

// ---- block weights ---------------------------------------------------------

// Elements of the staging buffer the weight upload goes through: the widest
// part of one layer, W1 [D][4D] or W2 [4D][D].
size_t block_stage_elems(int D) { return (size_t)4 * D * D; }

// Copy one layer's part at a time into `stage` (device, block_stage_elems(D)
// 16-bit values), then transpose it into the context's weight area; ends with
// a synchronisation of the stream.
fi_status load_block_weights(fi_ctx *c, const uint16_t *W, const uint16_t *W1, const uint16_t *W2, int on_device,
                             unsigned short *stage) {
    const int D = c->D, M = c->M;
    struct Part { const uint16_t *src; unsigned short *dst; int rows, cols; };
    const Part parts[3] = {{W, const_cast<unsigned short *>(c->dev.Wt), D, 3 * D},
                           {W1, const_cast<unsigned short *>(c->dev.W1t), D, 4 * D},
                           {W2, const_cast<unsigned short *>(c->dev.W2t), 4 * D, D}};
    hipError_t e = hipSuccess;
    for (int pi = 0; pi < 3 && e == hipSuccess; ++pi) {
        const Part &pt = parts[pi];
        const size_t per = (size_t)pt.rows * pt.cols;
        for (int l = 0; l < M && e == hipSuccess; ++l) {
            e = hipMemcpyAsync(stage, pt.src + l * per, per * sizeof(unsigned short),
                               on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, c->stream);
            if (e != hipSuccess) break;
            hipLaunchKernelGGL(k_transpose16, dim3((pt.cols + 31) / 32, (pt.rows + 31) / 32), dim3(256), 0,
                               c->stream, stage, pt.dst + l * per, pt.rows, pt.cols);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(c, FI_EDEVICE, std::string("block weights: ") + hipGetErrorString(e));
    c->weights_set = true;
    return FI_OK;
}

// Staging for fi_set_block_weights_static: a fixed device array instead of an
// allocation.  In host code `scratch` only names the symbol; its device
// address, one per device, comes from hipGetSymbolAddress and is kept here.
// Every call on a device shares that device's array: calls that overlap on one
// device (different streams or threads) race.
constexpr size_t kStaticStageBytes = size_t(4) * kBlockSpan * kBlockSpan * sizeof(unsigned short);
constexpr size_t kStaticStageElems = kStaticStageBytes / sizeof(unsigned short);
static __device__ __align__(256) unsigned short scratch[kStaticStageElems];
constexpr int kMaxDevices = 64;
std::mutex g_stage_mu;
void *g_stage_ptr[kMaxDevices] = {nullptr};

fi_status static_stage(fi_ctx *c, unsigned short **out) {
    int dev = -1;
    HIPCK(c, hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(c, FI_EDEVICE, "device index out of range for the static scratch");
    std::lock_guard<std::mutex> lock(g_stage_mu);
    if (!g_stage_ptr[dev]) {
        void *ptr = nullptr;
        HIPCK(c, hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return fail(c, FI_EDEVICE, "hipGetSymbolAddress returned no address for the static scratch");
        g_stage_ptr[dev] = ptr;
    }
    *out = (unsigned short *)g_stage_ptr[dev];
    return FI_OK;
}

// Whether fi_prefill may take the eager path (see fi_options.eager_prefill):
// every gray block after a position n <= P must have a prefill form.  Blocks
// of one-workgroup width may end anywhere (their targets past P go to the
// pending sums); two-half blocks must end inside the prompt (k_pre_fft2) or
// start at n = P; wider blocks must start at n = P (both run after the layer
// loop with the generation kernels, since their targets all lie past P).
bool eager_prefill_ok(const fi_ctx *c, int64_t P) {
    const int64_t G = c->dev.G;
    const int vlog = c->opt.fft_max_log2;
    if (!(c->opt.eager_prefill && c->pos == 0 && P > 0 && P < c->L && G >= 4 && G <= kPreNearMax && P % G == 0 &&
          (c->opt.map == FI_MAP_TANH || c->opt.map == FI_MAP_IDENTITY) && P <= c->pre_stride))
        return false;
    for (int q = ilog2_exact(G); (int64_t(1) << q) <= P; ++q) {
        const int64_t U = int64_t(1) << q;
        for (int64_t n = U; n <= P; n += 2 * U) {
            if (q <= vlog || n == P) continue;
            if (is_pair(q, vlog) && n + U <= P) continue;
            return false;
        }
    }
    return true;
}

// Two-half blocks of class q inside the prompt (n + 2^q <= P), layer l.
hipError_t launch_pre_fft2(fi_ctx *c, int q, int l, int64_t P) {
    const int logm = q - 1;
    const PreFftK k = pre_fft2_k(logm);
    if (!k) return hipErrorInvalidValue;
    const long long BD = (long long)c->B * c->D, pb = fft_per_block(logm);
    const unsigned nb = (unsigned)(((P >> q) + 1) >> 1);   // odd multiples of 2^q up to P
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)((BD + pb - 1) / pb), nb), dim3(fft_tpb(logm)), 0, c->stream, c->dev,
                       (const float4 *)c->spec[q], l, (long long)P, c->pre, c->pre_stride);
    return hipGetLastError();
}

hipError_t launch_pre_fft(fi_ctx *c, int q, int l, int64_t P) {
    const PreFftK k = pre_fft_k(q);
    if (!k) return hipErrorInvalidValue;
    const long long BD = (long long)c->B * c->D, pb = fft_per_block(q);
    const unsigned nb = (unsigned)(((P >> q) + 1) >> 1);   // odd multiples of 2^q up to P
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)((BD + pb - 1) / pb), nb), dim3(fft_tpb(q)), 0, c->stream, c->dev,
                       (const float4 *)c->spec[q], l, (long long)P, c->pre, c->pre_stride);
    return hipGetLastError();
}

// The prompt x[P][B][D] at position 0, layer by layer with all positions at
// once; leaves the state of P teacher-forced positions (ring rebuilt lazily).
fi_status eager_prefill(fi_ctx *c, const float *x, int64_t P, float *y) {
    const long long BD = (long long)c->B * c->D;
    const unsigned cells = (unsigned)((BD * P + 255) / 256);
    const int G = (int)c->dev.G, qg = ilog2_exact(G);
    hipLaunchKernelGGL(k_pre_in, dim3(cells), dim3(256), 0, c->stream, c->dev, x, (long long)P);
    HIPCK(c, hipGetLastError());
    for (int l = 0; l < c->M; ++l) {
        hipLaunchKernelGGL(k_pre_near, dim3((unsigned)(BD * (P / G))), dim3(kPreNearMax), 0, c->stream, c->dev, l,
                           (long long)P, G, c->pre, c->pre_stride);
        HIPCK(c, hipGetLastError());
        for (int q = qg; (int64_t(1) << q) <= P; ++q) {
            if (q <= c->opt.fft_max_log2) HIPCK(c, launch_pre_fft(c, q, l, P));
            else if (is_pair(q, c->opt.fft_max_log2)) HIPCK(c, launch_pre_fft2(c, q, l, P));
        }
        hipLaunchKernelGGL(k_pre_red, dim3(cells), dim3(256), 0, c->stream, c->dev, l, (long long)P,
                           (const float *)c->pre, c->pre_stride, y);
        HIPCK(c, hipGetLastError());
    }
    // the block after P itself when it is wider than one workgroup transform:
    // its targets all lie past the prompt, so every layer's block runs now,
    // with the kernels of a generation
    const int qp = ctz64(P);
    fi_status s = FI_OK;
    if (qp > c->opt.fft_max_log2) {
        if ((s = set_state_pos(c, P - 1)) != FI_OK) return s;
        HIPCK(c, launch_fft(c, rd_of(P), qp, c->stream, 0));
    }
    if ((s = set_state_pos(c, P)) != FI_OK) return s;
    c->pos = P;
    c->ring_stale = true;          // the next per-position launch rebuilds the ring
    return FI_OK;
}

}  // namespace

extern "C" {

fi_status fi_prefill(fi_ctx *c, const float *x, int64_t P, float *y) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (!x || P < 0) return FI_EINVAL;
    if (c->pos + P > c->L) return FI_ERANGE;
    if (c->opt.map == FI_MAP_EXTERNAL) return fail(c, FI_ESTATE, "fi_prefill in external-block mode");
    if (c->opt.map == FI_MAP_HYENA && !c->weights_set) return fail(c, FI_ESTATE, "block weights not set");
    if ((s = enter_mode(c, 1)) != FI_OK) return s;
    if (eager_prefill_ok(c, P)) return eager_prefill(c, x, P, y);
    const size_t BD = (size_t)c->B * c->D;
    const int64_t pos0 = c->pos, end = c->pos + P;
    while (c->pos < end) {
        const int64_t i = c->pos - pos0;
        if (chunk_fits(c, c->pos, end)) {
            const int64_t G = int64_t(1) << c->chunk_log;
            if ((s = join_side(c, c->pos + G)) != FI_OK) return s;
            if ((s = run_chunk(c, c->pos, x + i * BD)) != FI_OK) return s;
            if (y)
                HIPCK(c, hipMemcpyAsync(y + i * BD, c->dev.ylast + c->pos * BD, G * BD * sizeof(float),
                                        hipMemcpyDeviceToDevice, c->stream));
            c->pos += G;
            continue;
        }
        s = fi_step(c, x + i * BD, y ? y + i * BD : nullptr);
        if (s != FI_OK) return s;
    }
    return FI_OK;
}

fi_status fi_generate(fi_ctx *c, int64_t steps, float *y) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map == FI_MAP_EXTERNAL) return fail(c, FI_ESTATE, "fi_generate in external-block mode");
    if (c->opt.map == FI_MAP_HYENA && !c->weights_set) return fail(c, FI_ESTATE, "block weights not set");
    if (steps < 0) return FI_EINVAL;
    if (c->pos + steps > c->L) return FI_ERANGE;
    if ((s = enter_mode(c, 1)) != FI_OK) return s;
    const int64_t pos0 = c->pos, end = c->pos + steps;
    const int64_t bsize = c->block_log ? (int64_t(1) << c->block_log) : 0;
    const bool graphs = c->opt.use_graphs != 0;
    while (c->pos < end) {
        const int64_t n = c->pos + 1;
        if (chunk_fits(c, c->pos, end)) {
            // a split gray block deferred earlier feeds targets past side_until
            const int64_t G = int64_t(1) << c->chunk_log;
            if (graphs && !c->opt.time_blocks && c->gchunk[c->chunk_log]) {
                // an aligned run of 2^kb chunks: all but the last from one graph
                const int kb = c->chunk_block_log;
                const int64_t run = G << kb;
                const bool split_in_run = defers(c, c->chunk_log + kb - 1);
                if (kb && !split_in_run && (c->pos & (run - 1)) == 0 && c->pos + run <= end) {
                    if ((s = join_side(c, c->pos + run - G)) != FI_OK) return s;
                    HIPCK(c, hipGraphLaunch(c->gchunks, c->stream));
                    c->pos += run - G;
                    c->ring_stale = true;
                }
                const int64_t n = c->pos + G;
                const int q = class_of(c, n);
                if (!defers(c, q)) {
                    if ((s = join_side(c, n)) != FI_OK) return s;
                    HIPCK(c, hipGraphLaunch(c->gchunk[q], c->stream));
                    c->pos = n;
                    c->ring_stale = true;
                    continue;
                }
            }
            if ((s = join_side(c, c->pos + G)) != FI_OK) return s;
            if ((s = run_chunk(c, c->pos, nullptr)) != FI_OK) return s;
            c->pos += G;
            continue;
        }
        if ((s = join_side(c, n)) != FI_OK) return s;
        if ((s = resume_ring(c)) != FI_OK) return s;
        if (graphs && bsize && ((n - 1) & (bsize - 1)) == 0 && n + bsize - 2 <= end) {
            if ((s = join_side(c, n + bsize - 2)) != FI_OK) return s;
            HIPCK(c, hipGraphLaunch(c->gblock, c->stream));
            c->pos += bsize - 1;
            continue;
        }
        if ((s = join_side(c, n)) != FI_OK) return s;
        const int q = class_of(c, n);
        if (c->opt.time_blocks && q < c->P && c->path[q] == FI_PATH_FFT && c->opt.map != FI_MAP_HYENA) {
            s = launch_timed_position(c, n, q);
            if (s != FI_OK) return s;
        } else if (graphs && !(c->path[q] == FI_PATH_FFT && defers(c, q))) {
            HIPCK(c, hipGraphLaunch(c->gclass[q], c->stream));
        } else {
            // split gray blocks launch directly, leaving their later sub-blocks to the side stream
            HIPCK(c, launch_position(c, rd_of(n), q, c->stream, nullptr, nullptr, 1, n));
        }
        c->pos = n;
    }
    if (y && steps > 0) {
        const size_t BD = (size_t)c->B * c->D;
        HIPCK(c, hipMemcpyAsync(y, c->dev.ylast + pos0 * BD, steps * BD * sizeof(float),
                                hipMemcpyDeviceToDevice, c->stream));
    }
    return FI_OK;
}

fi_status fi_debug_schedule(const fi_ctx *c, int64_t n, int *q, int *path) {
    if (!c || n < 1 || n > c->L) return FI_EINVAL;
    const int cls = n < c->L ? ctz64(n) : -1;
    if (q) *q = cls;
    if (path) *path = cls < 0 ? FI_PATH_NONE : c->path[cls];
    return FI_OK;
}

fi_status fi_tau_table(const fi_ctx *c, int *path, double *us_direct, double *us_fft) {
    if (!c) return FI_EINVAL;
    for (int q = 0; q < c->P; ++q) {
        if (path) path[q] = c->path[q];
        if (us_direct) us_direct[q] = c->us_direct[q];
        if (us_fft) us_fft[q] = c->us_fft[q];
    }
    return FI_OK;
}

fi_status fi_chunk_table(const fi_ctx *c, double *us_chunk, double *us_run) {
    if (!c) return FI_EINVAL;
    for (int g = 0; g <= c->P; ++g) {
        if (us_chunk) us_chunk[g] = c->us_chunk[g];
        if (us_run) us_run[g] = c->us_run[g];
    }
    return FI_OK;
}

fi_status fi_history(const fi_ctx *cc, int layer, int what, int64_t first, int64_t count, float *dst) {
    fi_ctx *c = const_cast<fi_ctx *>(cc);
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (layer < 0 || layer >= c->M || first < 1 || count < 0 || first - 1 + count > c->L || !dst || what < 0 ||
        what > 2)
        return FI_EINVAL;
    if (!c->dev.recx) return fail(c, FI_ESTATE, "histories are recorded only with record = 1");
    if (what == 2 && !c->dev.reca) return fail(c, FI_ESTATE, "block outputs exist only with FI_MAP_HYENA");
    if (count == 0) return FI_OK;
    const size_t BD = (size_t)c->B * c->D;
    const float *src = (what == 0 ? c->dev.recx : what == 1 ? c->dev.recy : c->dev.reca) + (size_t)layer * BD +
                       (size_t)(first - 1) * c->M * BD;
    HIPCK(c, hipMemcpy2DAsync(dst, BD * sizeof(float), src, (size_t)c->M * BD * sizeof(float), BD * sizeof(float),
                              (size_t)count, hipMemcpyDeviceToDevice, c->stream));
    return FI_OK;
}

fi_status fi_set_block_weights(fi_ctx *c, const uint16_t *W, const uint16_t *W1, const uint16_t *W2,
                               int on_device) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map != FI_MAP_HYENA) return fail(c, FI_ESTATE, "block weights need FI_MAP_HYENA");
    if (!W || !W1 || !W2) return FI_EINVAL;
    unsigned short *tmp = nullptr;
    HIPCK(c, hipMalloc((void **)&tmp, block_stage_elems(c->D) * sizeof(unsigned short)));
    s = load_block_weights(c, W, W1, W2, on_device, tmp);
    (void)hipFree(tmp);
    return s;
}

fi_status fi_set_block_weights_static(fi_ctx *c, const uint16_t *W, const uint16_t *W1, const uint16_t *W2,
                                      int on_device) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map != FI_MAP_HYENA) return fail(c, FI_ESTATE, "block weights need FI_MAP_HYENA");
    if (!W || !W1 || !W2) return FI_EINVAL;
    if (block_stage_elems(c->D) > kStaticStageElems)
        return fail(c, FI_EINVAL,
                    "fi_set_block_weights_static: D = " + std::to_string(c->D) + " needs " +
                        std::to_string(block_stage_elems(c->D) * sizeof(unsigned short)) +
                        " bytes of staging, more than the " + std::to_string(kStaticStageBytes) +
                        " of the static scratch (D <= " + std::to_string(kBlockSpan) + ")");
    unsigned short *stage = nullptr;
    if ((s = static_stage(c, &stage)) != FI_OK) return s;
    return load_block_weights(c, W, W1, W2, on_device, stage);
}

fi_status fi_stamps(fi_ctx *c, int64_t first, int64_t count, int64_t *dst) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (first < 0 || count < 0 || first + count > c->L + 1 || (!dst && count)) return FI_EINVAL;
    HIPCK(c, hipStreamSynchronize(c->stream));
    if (count) {
        // the later of the two rows (the second is written only where a
        // position ends in several workgroups at once, zero elsewhere)
        std::vector<int64_t> second((size_t)count);
        HIPCK(c, hipMemcpy(dst, c->dev.stamps + first, count * sizeof(long long), hipMemcpyDeviceToHost));
        HIPCK(c, hipMemcpy(second.data(), c->dev.stamps + (c->L + 1) + first, count * sizeof(long long),
                           hipMemcpyDeviceToHost));
        for (int64_t k = 0; k < count; ++k) dst[k] = std::max(dst[k], second[(size_t)k]);
    }
    return FI_OK;
}

fi_status fi_layer_red(fi_ctx *c, int layer, const float *q, float *y) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map != FI_MAP_EXTERNAL) return fail(c, FI_ESTATE, "fi_layer_red needs FI_MAP_EXTERNAL");
    if (layer < 0 || layer >= c->M || !q || !y) return FI_EINVAL;
    if (c->pos >= c->L) return FI_ERANGE;
    if ((s = enter_mode(c, 1)) != FI_OK) return s;
    const int n = c->B * c->D;
    hipLaunchKernelGGL(k_red_layer, dim3((n + 255) / 256), dim3(256), 0, c->stream, c->dev, rd_of(c->pos + 1),
                       layer, q, y);
    HIPCK(c, hipGetLastError());
    return FI_OK;
}

fi_status fi_tiles(fi_ctx *c) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map != FI_MAP_EXTERNAL) return fail(c, FI_ESTATE, "fi_tiles needs FI_MAP_EXTERNAL");
    if (c->pos >= c->L) return FI_ERANGE;
    const int64_t n = c->pos + 1;
    if ((s = join_side(c, n)) != FI_OK) return s;
    HIPCK(c, launch_tiles(c, rd_of(n), class_of(c, n), c->stream, n));
    c->pos = n;
    return FI_OK;
}

fi_status fi_lazy_step(fi_ctx *c, const float *x_t, float *y_t) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (c->opt.map == FI_MAP_EXTERNAL || c->opt.map == FI_MAP_HYENA)
        return fail(c, FI_ESTATE, "Lazy path needs an elementwise map");
    if (c->pos >= c->L) return FI_ERANGE;
    if ((s = enter_mode(c, 2)) != FI_OK) return s;
    const int rd = rd_of(c->pos + 1);
    HIPCK(c, launch_baseline(c, FI_BASE_LAZY, rd, c->pos + 1, x_t, y_t, 1));
    c->pos += 1;
    return FI_OK;
}

fi_status fi_baseline_step(fi_ctx *c, int kind, const float *x_t, float *y_t) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (kind < FI_BASE_LAZY || kind > FI_BASE_EAGER_NP) return FI_EINVAL;
    if (c->opt.map == FI_MAP_EXTERNAL || c->opt.map == FI_MAP_HYENA)
        return fail(c, FI_ESTATE, "the baselines need an elementwise map");
    if (c->pos >= c->L) return FI_ERANGE;
    const bool eager = kind == FI_BASE_EAGER || kind == FI_BASE_EAGER_NP;
    if ((s = enter_mode(c, eager ? 4 : 2)) != FI_OK) return s;
    const int rd = rd_of(c->pos + 1);
    HIPCK(c, launch_baseline(c, kind, rd, c->pos + 1, x_t, y_t, 1));
    c->pos += 1;
    return FI_OK;
}

fi_status fi_baseline_generate(fi_ctx *c, int kind, int64_t steps, float *y) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (steps < 0) return FI_EINVAL;
    if (c->pos + steps > c->L) return FI_ERANGE;
    const int64_t pos0 = c->pos;
    for (int64_t i = 0; i < steps; ++i) {
        s = fi_baseline_step(c, kind, nullptr, nullptr);
        if (s != FI_OK) return s;
    }
    if (y && steps > 0) {
        const size_t BD = (size_t)c->B * c->D;
        HIPCK(c, hipMemcpyAsync(y, c->dev.ylast + pos0 * BD, steps * BD * sizeof(float),
                                hipMemcpyDeviceToDevice, c->stream));
    }
    return FI_OK;
}

fi_status fi_baseline_time(fi_ctx *c, int kind, int64_t n, int reps, double *us) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = join_side(c, -1)) != FI_OK) return s;
    if (kind < FI_BASE_LAZY || kind > FI_BASE_EAGER_NP) return FI_EINVAL;
    if (n < 1 || n > c->L || reps < 1 || !us) return FI_EINVAL;
    if (c->opt.map == FI_MAP_EXTERNAL || c->opt.map == FI_MAP_HYENA)
        return fail(c, FI_ESTATE, "the baselines need an elementwise map");
    if ((s = set_state_pos(c, n - 1)) != FI_OK) return s;
    c->mode = 3;  // rows now hold timing garbage: only fi_reset leaves this mode
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    const int rd = rd_of(n);
    HIPCK(c, launch_baseline(c, kind, rd, n, nullptr, nullptr, 0));  // warm-up
    HIPCK(c, hipEventRecord(a, c->stream));
    for (int r = 0; r < reps; ++r) HIPCK(c, launch_baseline(c, kind, rd, n, nullptr, nullptr, 0));
    HIPCK(c, hipEventRecord(b, c->stream));
    HIPCK(c, hipEventSynchronize(b));
    float ms = 0.f;
    HIPCK(c, hipEventElapsedTime(&ms, a, b));
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    *us = ms * 1000.0 / reps;
    return FI_OK;
}

fi_status fi_block_times(fi_ctx *c, int clear, double *ms, int64_t *count) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = harvest_events(c)) != FI_OK) return s;
    for (int q = 0; q < c->P; ++q) {
        if (ms) ms[q] = c->blk_ms[q];
        if (count) count[q] = c->blk_count[q];
        if (clear) {
            c->blk_ms[q] = 0.0;
            c->blk_count[q] = 0;
        }
    }
    return FI_OK;
}

fi_status fi_chunk_times(fi_ctx *c, int clear, double *ms, int64_t *count) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = harvest_events(c)) != FI_OK) return s;
    if (ms) *ms = c->chunk_ms;
    if (count) *count = c->chunk_count;
    if (clear) {
        c->chunk_ms = 0.0;
        c->chunk_count = 0;
    }
    return FI_OK;
}

fi_status fi_time_block(fi_ctx *c, int q, int path, int reps, double *us) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = join_side(c, -1)) != FI_OK) return s;
    if (q < 0 || q >= c->P || reps < 1 || !us) return FI_EINVAL;
    if (path == FI_PATH_DIRECT ? !direct_exists(q) : path == FI_PATH_FFT ? !fft_exists(q, c->P) : true)
        return FI_EINVAL;
    const int64_t n = int64_t(1) << q;
    if ((s = set_state_pos(c, n - 1)) != FI_OK) return s;
    c->mode = 3;  // rows now hold timing garbage: only fi_reset leaves this mode
    const int rd = rd_of(n);
    auto once = [&]() -> hipError_t {
        return path == FI_PATH_DIRECT ? launch_direct<true>(c, rd, q, c->stream, nullptr, nullptr, 0)
                                      : launch_fft(c, rd, q, c->stream, 0);
    };
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    HIPCK(c, once());  // warm-up
    HIPCK(c, hipEventRecord(a, c->stream));
    for (int r = 0; r < reps; ++r) HIPCK(c, once());
    HIPCK(c, hipEventRecord(b, c->stream));
    HIPCK(c, hipEventSynchronize(b));
    float ms = 0.f;
    HIPCK(c, hipEventElapsedTime(&ms, a, b));
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    *us = ms * 1000.0 / reps;
    return FI_OK;
}

fi_status fi_time_hyena_block(fi_ctx *c, int reps, double *us) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = join_side(c, -1)) != FI_OK) return s;
    if (reps < 1 || !us) return FI_EINVAL;
    if (c->opt.map != FI_MAP_HYENA) return fail(c, FI_ESTATE, "fi_time_hyena_block needs FI_MAP_HYENA");
    if (!c->weights_set) return fail(c, FI_ESTATE, "block weights not set");
    if ((s = set_state_pos(c, 0)) != FI_OK) return s;
    c->mode = 3;  // rows now hold timing garbage: only fi_reset leaves this mode
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    HIPCK(c, launch_hyena_block(c, 0, c->stream, nullptr, nullptr));  // warm-up
    HIPCK(c, hipEventRecord(a, c->stream));
    for (int r = 0; r < reps; ++r) HIPCK(c, launch_hyena_block(c, 0, c->stream, nullptr, nullptr));
    HIPCK(c, hipEventRecord(b, c->stream));
    HIPCK(c, hipEventSynchronize(b));
    float ms = 0.f;
    HIPCK(c, hipEventElapsedTime(&ms, a, b));
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    *us = ms * 1000.0 / reps;
    return FI_OK;
}

fi_status fi_lazy_time(fi_ctx *c, int64_t n, int reps, double *us) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if ((s = join_side(c, -1)) != FI_OK) return s;
    if (n < 1 || n > c->L || reps < 1 || !us) return FI_EINVAL;
    if (c->opt.map == FI_MAP_EXTERNAL || c->opt.map == FI_MAP_HYENA)
        return fail(c, FI_ESTATE, "Lazy path needs an elementwise map");
    if ((s = set_state_pos(c, n - 1)) != FI_OK) return s;
    c->mode = 3;  // rows now hold timing garbage: only fi_reset leaves this mode
    hipEvent_t a, b;
    HIPCK(c, hipEventCreate(&a));
    HIPCK(c, hipEventCreate(&b));
    const int rd = rd_of(n);
    auto once = [&]() -> hipError_t { return launch_baseline(c, FI_BASE_LAZY, rd, n, nullptr, nullptr, 0); };
    HIPCK(c, once());  // warm-up
    HIPCK(c, hipEventRecord(a, c->stream));
    for (int r = 0; r < reps; ++r) HIPCK(c, once());
    HIPCK(c, hipEventRecord(b, c->stream));
    HIPCK(c, hipEventSynchronize(b));
    float ms = 0.f;
    HIPCK(c, hipEventElapsedTime(&ms, a, b));
    HIPCK(c, hipEventDestroy(a));
    HIPCK(c, hipEventDestroy(b));
    *us = ms * 1000.0 / reps;
    return FI_OK;
}

fi_status fi_lazy_generate(fi_ctx *c, int64_t steps, float *y) {
    fi_status s = check_usable(c);
    if (s != FI_OK) return s;
    if (steps < 0) return FI_EINVAL;
    if (c->pos + steps > c->L) return FI_ERANGE;
    const int64_t pos0 = c->pos;
    for (int64_t i = 0; i < steps; ++i) {
        s = fi_lazy_step(c, nullptr, nullptr);
        if (s != FI_OK) return s;
    }
    if (y && steps > 0) {
        const size_t BD = (size_t)c->B * c->D;
        HIPCK(c, hipMemcpyAsync(y, c->dev.ylast + pos0 * BD, steps * BD * sizeof(float),
                                hipMemcpyDeviceToDevice, c->stream));
    }
    return FI_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Data-dependent filters: the taps arrive with the data (fi_dd_*).
// ---------------------------------------------------------------------------
struct fi_dd {
    int M = 1;                       // layers (a stack: rows r = l * B * D + b * D + c)
    bool stack = false;              // made by fi_dd_stack_init: red cells through the layers first
    float *xs = nullptr;             // a stack's layer inputs of the current position [M][B][D]
    int B = 0, D = 0, R = 0, kmin = 0, kmax = -1;
    int64_t L = 0, pos = 0;
    hipStream_t stream = nullptr;
    char *ws = nullptr;
    fi::Dev dev{};
    fi::DDev q{};
    float4 *spx[kMaxP] = {}, *sph[kMaxP] = {};
    bool poisoned = false;
    std::string err;
};

namespace {

constexpr int kDDMaxLog = 15;      // L <= 2^15: the widest product (L/2) is one workgroup's transform
constexpr int kDDFftMinDefault = 8;    // products of p <= 128 run in the per-position launch

struct DDLayout {
    size_t xh = 0, hh = 0, acc = 0, twid = 0, xs = 0, total = 0;
    size_t spx[kMaxP] = {0}, sph[kMaxP] = {0};
    int kmin = 0, kmax = -1, logNT = 2;
};

bool dd_layout(int B, int D, int64_t L, int fft_min, DDLayout &ly) {
    if (B < 1 || D < 1 || L < 1 || L > (int64_t(1) << kDDMaxLog) || (L & (L - 1)) != 0 ||
        (int64_t)B * D > (int64_t(1) << 24))
        return false;
    if (fft_min < 2 || fft_min > kDDMaxLog) return false;
    const size_t R = (size_t)B * D;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    ly.xh = take(R * L * sizeof(float));
    ly.hh = take(R * L * sizeof(float));
    ly.acc = take(R * L * sizeof(float));
    ly.kmin = fft_min;
    ly.kmax = -1;
    for (int k = fft_min; (int64_t(2) << k) <= L; ++k) ly.kmax = k;   // products of p = 2^k: 2p <= L
    for (int k = ly.kmin; k <= ly.kmax; ++k) {
        ly.spx[k] = take(R * (size_t(1) << (k - 1)) * sizeof(float4));
        ly.sph[k] = take(R * (size_t(1) << (k - 1)) * sizeof(float4));
    }
    ly.logNT = std::max(2, ly.kmax + 1);
    ly.twid = take((size_t(2) << ly.logNT) * sizeof(float2));
    ly.xs = take(R * sizeof(float));
    ly.total = off;
    return true;
}

// A stack of M layers: the rows of every layer in one context (R = M B D).
bool dd_stack_layout(int M, int B, int D, int64_t L, int fft_min, DDLayout &ly) {
    if (M < 1 || M > kMaxLayers || (int64_t)M * B > (int64_t(1) << 24)) return false;
    return dd_layout(M * B, D, L, fft_min, ly);
}

fi_status dd_fail(fi_dd *c, fi_status s, const std::string &msg) {
    c->err = msg;
    if (s == FI_EDEVICE) c->poisoned = true;
    return s;
}

#define DDCK(ctx, call)                                                                      \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return dd_fail((ctx), FI_EDEVICE, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

void dd_launch(fi_dd *c, int k, int64_t n) {
    const fi::DDBandK kb = fi::dd_band_k(k);
    const fi::DDFftK kf = fi::dd_fft_k(k);
    if (!kb || !kf) return;
    const long long pb = fft_per_block(k);
    const unsigned grid = (unsigned)((c->R + pb - 1) / pb);
    if (n + 1 == (int64_t(2) << k))   // the fixed blocks x[p, 2p), h[p, 2p) are complete: their spectra
        hipLaunchKernelGGL(kb, dim3(grid, 2), dim3(fft_tpb(k)), 0, c->stream, c->dev, c->q, c->spx[k], c->sph[k]);
    hipLaunchKernelGGL(kf, dim3(grid), dim3(fft_tpb(k)), 0, c->stream, c->dev, c->q, (const float4 *)c->spx[k],
                       (const float4 *)c->sph[k], (long long)n);
}

void dd_near_launch(fi_dd *c, int pm, int64_t n, const float *x, const float *h, float *y, bool prod) {
    const int rpw = 128 / pm;   // rows per 256-thread workgroup
    hipLaunchKernelGGL(fi::dd_near_k(pm), dim3((unsigned)((c->R + rpw - 1) / rpw)), dim3(256), 0, c->stream, c->q,
                       (long long)n, x, h, y, prod);
}

fi_status dd_step(fi_dd *c, const float *x, const float *h, float *y) {
    const int64_t n = c->pos;
    if (c->stack) {
        // a stack: the red cells layer after layer, then every layer's products from the staged inputs
        const int BD = c->B * c->D;
        hipLaunchKernelGGL(fi::k_dd_chain, dim3((unsigned)((BD + 255) / 256)), dim3(256), 0, c->stream, c->q, c->M,
                           BD, (long long)n, x, h, y, c->xs);
        x = c->xs;
    }
    // largest direct product of this position up to the one-launch limit (0: none)
    int64_t pm = 0;
    for (int64_t p = 1; p <= fi::kDDNearMax && p < c->q.pd && 2 * p <= n + 1 && (n + 1) % p == 0; p *= 2) pm = p;
    dd_near_launch(c, pm ? (int)pm : 1, n, x, h, y, pm != 0);
    const int64_t pw = 2 * fi::kDDNearMax;
    if (c->q.pd > pw && 2 * pw <= n + 1 && (n + 1) % pw == 0)
        hipLaunchKernelGGL(fi::k_dd_wide, dim3((unsigned)((c->R + 255) / 256)), dim3(256), 0, c->stream, c->q,
                           (long long)n);
    for (int k = c->kmin; k <= c->kmax && (int64_t(2) << k) <= n + 1 && (n + 1) % (int64_t(1) << k) == 0; ++k)
        dd_launch(c, k, n);
    DDCK(c, hipGetLastError());
    ++c->pos;
    return FI_OK;
}

}  // namespace

extern "C" {

size_t fi_dd_workspace_bytes(int batch, int channels, int64_t L, int fft_min_log2) {
    DDLayout ly;
    return dd_layout(batch, channels, L, fft_min_log2 < 0 ? kDDFftMinDefault : fft_min_log2, ly) ? ly.total : 0;
}

}  // extern "C"

namespace {

fi_status dd_init(fi_dd **out, bool stack, int layers, int batch, int channels, int64_t L, int fft_min_log2,
                  void *workspace, void *stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    if (!out || !workspace) return FI_EINVAL;
    *out = nullptr;
    DDLayout ly;
    if (!dd_stack_layout(layers, batch, channels, L, fft_min_log2 < 0 ? kDDFftMinDefault : fft_min_log2, ly))
        return FI_EINVAL;
    fi_dd *c = new fi_dd();
    c->M = layers;
    c->stack = stack;
    c->B = batch;
    c->D = channels;
    c->R = layers * batch * channels;
    c->L = L;
    c->stream = stream;
    c->ws = (char *)workspace;
    c->kmin = ly.kmin;
    c->kmax = ly.kmax;
    c->xs = (float *)(c->ws + ly.xs);
    c->q.xh = (float *)(c->ws + ly.xh);
    c->q.hh = (float *)(c->ws + ly.hh);
    c->q.acc = (float *)(c->ws + ly.acc);
    c->q.L = L;
    c->q.R = c->R;
    c->q.pd = 1 << ly.kmin;
    for (int k = ly.kmin; k <= ly.kmax; ++k) {
        c->spx[k] = (float4 *)(c->ws + ly.spx[k]);
        c->sph[k] = (float4 *)(c->ws + ly.sph[k]);
    }
    c->dev.twid = (const float2 *)(c->ws + ly.twid);
    c->dev.ptw = c->dev.twid + (size_t(1) << ly.logNT);
    c->dev.optw = c->dev.ptw + (size_t(1) << (ly.logNT - 1));
    c->dev.logNT = ly.logNT;
    const std::vector<float2> tw = twiddle_tables(ly.logNT);
    fi_status s = FI_OK;
    if (hipMemcpyAsync((void *)c->dev.twid, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice, stream) !=
            hipSuccess ||
        hipMemsetAsync(c->ws + ly.xh, 0, ly.twid - ly.xh, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        s = FI_EDEVICE;
    if (s != FI_OK) {
        delete c;
        return s;
    }
    *out = c;
    return FI_OK;
}

}  // namespace

extern "C" {

fi_status fi_dd_init(fi_dd **out, int batch, int channels, int64_t L, int fft_min_log2, void *workspace,
                     void *stream) {
    return dd_init(out, false, 1, batch, channels, L, fft_min_log2, workspace, stream);
}

size_t fi_dd_stack_workspace_bytes(int layers, int batch, int channels, int64_t L, int fft_min_log2) {
    DDLayout ly;
    return dd_stack_layout(layers, batch, channels, L, fft_min_log2 < 0 ? kDDFftMinDefault : fft_min_log2, ly)
               ? ly.total
               : 0;
}

fi_status fi_dd_stack_init(fi_dd **out, int layers, int batch, int channels, int64_t L, int fft_min_log2,
                           void *workspace, void *stream) {
    return dd_init(out, true, layers, batch, channels, L, fft_min_log2, workspace, stream);
}

fi_status fi_dd_step(fi_dd *c, const float *x_t, const float *h_t, float *y_t) {
    if (!c || !x_t || !h_t || !y_t) return FI_EINVAL;
    if (c->poisoned) return FI_ESTATE;
    if (c->pos >= c->L) return dd_fail(c, FI_ERANGE, "stepped past L");
    return dd_step(c, x_t, h_t, y_t);
}

fi_status fi_dd_run(fi_dd *c, const float *x, const float *h, int64_t steps, float *y) {
    if (!c || steps < 0 || (steps > 0 && (!x || !h || !y))) return FI_EINVAL;
    if (c->poisoned) return FI_ESTATE;
    if (c->pos + steps > c->L) return dd_fail(c, FI_ERANGE, "run past L");
    const size_t R = (size_t)c->R, BD = (size_t)c->B * c->D;
    for (int64_t i = 0; i < steps; ++i) {
        const fi_status s = dd_step(c, x + i * BD, h + i * R, y + i * R);
        if (s != FI_OK) return s;
    }
    return FI_OK;
}

fi_status fi_dd_reset(fi_dd *c) {
    if (!c) return FI_EINVAL;
    if (c->poisoned) return FI_ESTATE;
    const size_t bytes = (size_t)c->R * c->L * sizeof(float);
    DDCK(c, hipMemsetAsync(c->q.xh, 0, bytes, c->stream));
    DDCK(c, hipMemsetAsync(c->q.hh, 0, bytes, c->stream));
    DDCK(c, hipMemsetAsync(c->q.acc, 0, bytes, c->stream));
    c->pos = 0;
    return FI_OK;
}

int64_t fi_dd_position(const fi_dd *c) { return c ? c->pos : -1; }

const char *fi_dd_last_error(const fi_dd *c) { return c ? c->err.c_str() : "null context"; }

fi_status fi_dd_destroy(fi_dd *c) {
    if (!c) return FI_OK;
    const hipError_t e = hipStreamSynchronize(c->stream);
    delete c;
    return e == hipSuccess ? FI_OK : FI_EDEVICE;
}

}  // extern "C"
