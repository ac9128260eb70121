// The tanh of the chunk kernels' red-cell chains (csrc/fi_tanh.h,
// tanh_chain), compiled for the CPU: its error against tanh in long double over
// every 7th float of [2^-30, 12], both signs, and over every float of
// [2^-30, 0.125) (the first piece).  The hardware exponential and reciprocal
// are replaced by the C library's, so this checks the formulas, the
// polynomials and the branch points; on the GPU each adds about 1 ulp more.
// Also: the cheaper passes of the chains give the same bits as tanh_chain on
// the ranges they are kept for (tanh_small below 0.72, tanh_tiny below 0.125),
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
    long n = 0, small_diff = 0, tiny_diff = 0, odd_diff = 0;
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
            if (y < fi::kTanhTiny) {
                const float alt = fi::tanh_tiny(v);
                if (std::memcmp(&alt, &got, 4) != 0) ++tiny_diff;
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
    // the first piece over every float of its range (one sign: the piece is
    // odd in its form), and its agreement with tanh_chain there
    float t0 = std::ldexp(1.0f, -30), t1 = fi::kTanhTiny;
    uint32_t tlo, thi;
    std::memcpy(&tlo, &t0, 4);
    std::memcpy(&thi, &t1, 4);
    double worst_tiny = 0, at_tiny = 0;
    for (uint32_t b = tlo; b < thi; ++b) {
        float y;
        std::memcpy(&y, &b, 4);
        const float got = fi::tanh_tiny(y);
        const long double ref = tanhl((long double)y);
        const double e = (double)std::fabs((long double)got - ref) / ulp_of((float)ref);
        if (e > worst_tiny) worst_tiny = e, at_tiny = y;
        const float full = fi::tanh_chain(y);
        if (std::memcmp(&full, &got, 4) != 0) ++tiny_diff;
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
                "every float below 0.125: %.3f ulp (at %.8g); saturation %s; tanh_small differs at %ld points "
                "below 0.72, tanh_tiny at %ld below 0.125; not odd at %ld points\n", n, worst_small, at_small,
                worst_big, at_big, worst_tiny, at_tiny, sat ? "ok" : "WRONG", small_diff, tiny_diff, odd_diff);
    return (worst_small <= 1.0 && worst_big <= 1.6 && worst_tiny <= 0.7 && sat && small_diff == 0 &&
            tiny_diff == 0 && odd_diff == 0)
               ? 0
               : 1;
}
