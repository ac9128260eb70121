// host shim for tests/kernel_math: the few HIP names fi_fft.h uses, for a CPU build
// host shim: just enough of the HIP vector types to compile the FFT header on the CPU
#pragma once
#include <cmath>
#include <cstdint>
#include <cstddef>
#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __launch_bounds__(x)
#define __restrict__
struct float2 { float x, y; };
struct float4 { float x, y, z, w; };
inline float2 make_float2(float a, float b) { return {a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline uint64_t wall_clock64() { return 0; }
inline unsigned atomicAdd(unsigned* p, unsigned v) { unsigned o = *p; *p += v; return o; }
inline void __syncthreads() {}
struct dim3_ { unsigned x = 0, y = 0, z = 0; };
static dim3_ threadIdx, blockIdx, blockDim, gridDim;
// hardware base-2 exponential and reciprocal: the C library's stand-ins
#define __builtin_amdgcn_exp2f(x) std::exp2((float)(x))
#define __builtin_amdgcn_rcpf(x) (1.0f / (float)(x))
