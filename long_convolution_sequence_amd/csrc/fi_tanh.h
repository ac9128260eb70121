// The tanh of the chunk kernels' red-cell chains (fi_chunk.h).  Kept apart
// from the device helpers that every kernel includes, so that it can change
// without touching them, and compiled for the CPU by tests/kernel_math.
#pragma once
#include <hip/hip_runtime.h>

namespace fi {

// tanh without branches, for the red-cell chains (the critical path of a
// chunk of positions), in three pieces, all evaluated in y itself (odd, so no
// sign fix-up):
//   |y| < 0.125:  y + y^3 (c0 + c1 y^2)   (four operations; 0.63 ulp over every
//                 float of the range)
//   |y| < 0.72:   y + y^3 P(y^2), P of degree 4 in Horner's form (seven)
//   otherwise:    1 - 2 / (e^{2|y|} + 1), with e^{2|y|} from the hardware
//                 base-2 exponential and the reciprocal (where this difference
//                 cancels, below 0.72, the polynomials take over)
// The polynomials are fitted for least relative error (Lawson's iteratively
// reweighted least squares, in double on Chebyshev nodes; coefficients rounded
// to float).  A chain's wave runs alone on its SIMD and issues every operation
// of the layer, so the count of operations, not the depth of their
// dependences, sets the time per layer: the chains run the cheapest piece that
// covers the whole wave (see chain_run), and each function below gives the
// same bits as tanh_chain on its range.  Error under 1 ulp below 0.72.  Every
// piece is evaluated and one selected, so lanes on either side never diverge.
constexpr float kTanhTiny = 0.125f;             // the first piece's range, |y| < kTanhTiny
constexpr float kTanhTinySq = 0x1p-6f;          // 0.125^2, a float: y*y < this exactly when |y| < 0.125
constexpr float kTanhSmall = 0.72f;             // the polynomial pieces' range, |y| < kTanhSmall
constexpr float kTanhSmallSq = 0x1.096bbap-1f;  // 0.72f * 0.72f rounded: y*y < this exactly when |y| < 0.72f
__device__ __forceinline__ float tanh_tiny_p(float s) {   // c0 + c1 s
    return fmaf(s, 0.13216736912727356f, -0.3333277106285095f);
}
__device__ __forceinline__ float tanh_tiny(float y) {     // meaningful for |y| < 0.125
    const float s = y * y;
    return fmaf(y * s, tanh_tiny_p(s), y);
}
__device__ __forceinline__ float tanh_small(float y) {    // both polynomial pieces; meaningful for |y| < 0.72
    const float s = y * y;
    float q = fmaf(s, -0.004989919252693653f, 0.01992698572576046f);
    q = fmaf(q, s, -0.05349649116396904f);
    q = fmaf(q, s, 0.13328194618225098f);
    q = fmaf(q, s, -0.33333149552345276f);
    q = s < kTanhTinySq ? tanh_tiny_p(s) : q;
    return fmaf(y * s, q, y);
}
// The full tanh: equal to tanh_small(y) for |y| < 0.72 and to tanh_tiny(y) for
// |y| < 0.125 (bit for bit).
__device__ __forceinline__ float tanh_chain(float y) {
    const float a = fabsf(y);
    const float e = __builtin_amdgcn_exp2f(a * 2.88539008f);      // e^{2a} = 2^{2a log2(e)}
    const float big = copysignf(fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f), y);
    const float small = tanh_small(y);
    return a < kTanhSmall ? small : big;
}

}  // namespace fi
