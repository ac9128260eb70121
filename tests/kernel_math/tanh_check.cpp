// The tanh of the chunk kernels' red-cell chains (csrc/fi_tanh.h,
// tanh_chain), compiled for the CPU: its error against tanh in long double over
// every 7th float of [2^-30, 12], both signs.  The hardware exponential and
// reciprocal are replaced by the C library's, so this checks the formula, the
// polynomial and the branch point; on the GPU each adds about 1 ulp more.
// Also: the polynomial half alone (tanh_small, the chains' first pass) gives
// the same bits as tanh_chain wherever |y| < 0.72, the range it is kept for,
// and the result is odd bit for bit (tanh(-y) = -tanh(y)).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hip/hip_runtime.h"
#include "../../long_convolution_sequence_amd/csrc/fi_tanh.h"

static double ulp_of(float v) {
    const float a = std::fabs(v);
    return (double)std::nextafter(a, INFINITY) - (double)a;
}

int main() {
    uint32_t lo, hi;
    float f = std::ldexp(1.0f, -30), g = 12.0f;
    std::memcpy(&lo, &f, 4);
    std::memcpy(&hi, &g, 4);
    double worst_small = 0, worst_big = 0, at_small = 0, at_big = 0;
    long n = 0, small_diff = 0, odd_diff = 0;
    for (uint32_t b = lo; b <= hi; b += 7) {
        float y;
        std::memcpy(&y, &b, 4);
        for (int sgn = 0; sgn < 2; ++sgn) {
            const float v = sgn ? -y : y;
            const float got = fi::tanh_chain(v);
            if (sgn) {
                const float pos = fi::tanh_chain(y);
                if (!(got == -pos)) ++odd_diff;
            }
            if (y < fi::kTanhSmall) {
                const float alt = fi::tanh_small(v);
                if (std::memcmp(&alt, &got, 4) != 0) ++small_diff;
            }
            const long double ref = tanhl((long double)v);
            const double e = (double)std::fabs((long double)got - ref) / ulp_of((float)ref);
            if (y < fi::kTanhSmall) {
                if (e > worst_small) worst_small = e, at_small = v;
            } else if (e > worst_big) {
                worst_big = e, at_big = v;
            }
            ++n;
        }
    }
    // saturation; zero maps to zero (the odd-form polynomial gives +0 for -0: the
    // values are equal, and nothing downstream tells them apart), and the
    // smallest magnitudes keep their sign and value
    const float tiny = std::ldexp(1.0f, -140);
    const bool sat = fi::tanh_chain(60.f) == 1.f && fi::tanh_chain(-60.f) == -1.f &&
                     fi::tanh_chain(INFINITY) == 1.f && fi::tanh_chain(-INFINITY) == -1.f &&
                     fi::tanh_chain(-0.f) == 0.f && fi::tanh_chain(0.f) == 0.f &&
                     fi::tanh_chain(-tiny) == -tiny && fi::tanh_chain(tiny) == tiny;
    std::printf("tanh_chain: %ld points; |y| < 0.72: %.3f ulp (at %.8g); |y| >= 0.72: %.3f ulp (at %.8g); "
                "saturation %s; tanh_small differs at %ld points below 0.72; not odd at %ld points\n", n, worst_small,
                at_small, worst_big, at_big, sat ? "ok" : "WRONG", small_diff, odd_diff);
    return (worst_small <= 1.0 && worst_big <= 1.6 && sat && small_diff == 0 && odd_diff == 0) ? 0 : 1;
}
