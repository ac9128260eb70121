// The tanh of the chunk kernels' red-cell chains (fi_chunk.h).  Kept apart
// from the device helpers that every kernel includes, so that it can change
// without touching them, and compiled for the CPU by tests/kernel_math.
#pragma once
#include <hip/hip_runtime.h>

namespace fi {

// tanh without branches, for the red-cell chains (the critical path of a
// chunk of positions).  |y| >= 0.72: 1 - 2 / (e^{2|y|} + 1), with e^{2|y|}
// from the hardware base-2 exponential and the reciprocal.  |y| < 0.72, where
// that difference cancels: y + y^3 P(y^2), P of degree 4 fitted for least
// relative error (Lawson's iteratively reweighted least squares, in double on
// Chebyshev nodes; coefficients rounded to float).  P is evaluated in Horner's
// form and the result formed in y itself (odd, so no sign fix-up): seven
// operations in all.  A chain's wave runs alone on its SIMD and issues every
// operation of the layer, so the count of operations, not the depth of their
// dependences, sets the time per layer (degree 5 on |y| < 0.8 costs one more
// per layer).  Error under 1 ulp.  Both halves are evaluated and one selected,
// so lanes on either side never diverge.
constexpr float kTanhSmall = 0.72f;             // the polynomial half's range, |y| < kTanhSmall
constexpr float kTanhSmallSq = 0x1.096bbap-1f;  // 0.72f * 0.72f rounded: y*y < this exactly when |y| < 0.72f
__device__ __forceinline__ float tanh_small(float y) {   // y + y^3 P(y^2); meaningful for |y| < 0.72
    const float s = y * y;
    float q = fmaf(s, -0.004989919252693653f, 0.01992698572576046f);
    q = fmaf(q, s, -0.05349649116396904f);
    q = fmaf(q, s, 0.13328194618225098f);
    q = fmaf(q, s, -0.33333149552345276f);
    return fmaf(y * s, q, y);
}
// The full tanh: equal to tanh_small(y) for |y| < 0.72 (bit for bit).
__device__ __forceinline__ float tanh_chain(float y) {
    const float a = fabsf(y);
    const float e = __builtin_amdgcn_exp2f(a * 2.88539008f);      // e^{2a} = 2^{2a log2(e)}
    const float big = copysignf(fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f), y);
    const float small = tanh_small(y);
    return a < kTanhSmall ? small : big;
}

}  // namespace fi
