// Kernel-pointer tables of the kernel families with many compile-time
// variants.  Each family is instantiated in a translation unit of its own
// (fi_tab_*.hip) so the variants compile in parallel; the host code launches
// them through the pointers returned here (the HIP runtime registers every
// kernel of every translation unit under its host stub, so a kernel may be
// launched from any of them).  nullptr: no such variant.
#pragma once
#include <hip/hip_runtime.h>

#include "fi_device.h"

namespace fi {

struct DDev;

using FftTileK = void (*)(Dev, int, const float4 *, int);                    // k_fft_tile, k_fft_tile2
using SpectrumK = void (*)(Dev, float4 *, long long, long long);             // k_spectrum, k_spectrum2
using SubFwdK = void (*)(Dev, int, float4 *, int);                           // k_fft_sub_fwd
using SubInvK = void (*)(Dev, int, const float4 *, const float4 *, int, int, int, long long, int);
using PreFftK = void (*)(Dev, const float4 *, int, long long, float *, int);  // k_pre_fft
using ChunkK = void (*)(Dev, long long, int, int, const float *);            // k_chunk
using DDBandK = void (*)(Dev, DDev, float4 *, float4 *);                     // k_dd_band
using DDFftK = void (*)(Dev, DDev, const float4 *, const float4 *, long long);   // k_dd_fft
using DDNearK = void (*)(DDev, long long, const float *, const float *, float *, bool);  // k_dd_near

using HyProjK = void (*)(Dev, int, int, const float *);                      // k_hy_proj<B>
using HyStepK = void (*)(Dev, int, int);                                    // k_hy_up<B>, k_hy_down<B>

FftTileK fft_tile_k(int logn);     // one-workgroup transform, 2 <= logn <= 14
FftTileK fft_tile2_k(int logm);    // two halves of 2^logm, 12 <= logm <= 14
SubFwdK sub_fwd_k(int logv);       // split classes, sub-blocks of 2^logv, 12..14
SubInvK sub_inv_k(int logv, int K);   // K sub-blocks (a power of two, >= 4)
SpectrumK spectrum_k(int logn);    // 2..14
SpectrumK spectrum2_k(int logm);   // 12..14
PreFftK pre_fft_k(int logn);       // 2..14
PreFftK pre_fft2_k(int logm);      // two-half class of 2^(logm+1), 12..14
ChunkK chunk_k(int mt, int mode);  // mt = depth up to kChunkRegLayers, or 0; mode 0..3
DDBandK dd_band_k(int logp);       // 2..14
DDFftK dd_fft_k(int logp);         // 2..14
DDNearK dd_near_k(int pm);         // 1, 2, 4, .., 128
HyProjK hy_proj_k(int B);          // Hyena-style block kernels for batch B, 1 <= B <= 8
HyStepK hy_up_k(int B);
HyStepK hy_down_k(int B);

}  // namespace fi
