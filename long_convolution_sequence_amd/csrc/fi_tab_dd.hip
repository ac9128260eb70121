// Data-dependent-filter kernels with compile-time product sizes (see fi_tables.h).
#include "fi_tables.h"
#include "fi_dd_kernels.h"

namespace fi {

DDBandK dd_band_k(int logp) {
    switch (logp) {
        case 2: return &k_dd_band<2>;
        case 3: return &k_dd_band<3>;
        case 4: return &k_dd_band<4>;
        case 5: return &k_dd_band<5>;
        case 6: return &k_dd_band<6>;
        case 7: return &k_dd_band<7>;
        case 8: return &k_dd_band<8>;
        case 9: return &k_dd_band<9>;
        case 10: return &k_dd_band<10>;
        case 11: return &k_dd_band<11>;
        case 12: return &k_dd_band<12>;
        case 13: return &k_dd_band<13>;
        case 14: return &k_dd_band<14>;
        default: return nullptr;
    }
}

DDFftK dd_fft_k(int logp) {
    switch (logp) {
        case 2: return &k_dd_fft<2>;
        case 3: return &k_dd_fft<3>;
        case 4: return &k_dd_fft<4>;
        case 5: return &k_dd_fft<5>;
        case 6: return &k_dd_fft<6>;
        case 7: return &k_dd_fft<7>;
        case 8: return &k_dd_fft<8>;
        case 9: return &k_dd_fft<9>;
        case 10: return &k_dd_fft<10>;
        case 11: return &k_dd_fft<11>;
        case 12: return &k_dd_fft<12>;
        case 13: return &k_dd_fft<13>;
        case 14: return &k_dd_fft<14>;
        default: return nullptr;
    }
}

DDNearK dd_near_k(int pm) {
    switch (pm) {
        case 1: return &k_dd_near<1>;
        case 2: return &k_dd_near<2>;
        case 4: return &k_dd_near<4>;
        case 8: return &k_dd_near<8>;
        case 16: return &k_dd_near<16>;
        case 32: return &k_dd_near<32>;
        case 64: return &k_dd_near<64>;
        case 128: return &k_dd_near<128>;
        default: return nullptr;
    }
}

}  // namespace fi
