// Filter spectra and the eager prefill's FFT gray blocks (see fi_tables.h).
#include "fi_tables.h"
#include "fi_fft_kernels.h"

namespace fi {

SpectrumK spectrum_k(int logn) {
    switch (logn) {
        case 2: return &k_spectrum<2>;
        case 3: return &k_spectrum<3>;
        case 4: return &k_spectrum<4>;
        case 5: return &k_spectrum<5>;
        case 6: return &k_spectrum<6>;
        case 7: return &k_spectrum<7>;
        case 8: return &k_spectrum<8>;
        case 9: return &k_spectrum<9>;
        case 10: return &k_spectrum<10>;
        case 11: return &k_spectrum<11>;
        case 12: return &k_spectrum<12>;
        case 13: return &k_spectrum<13>;
        case 14: return &k_spectrum<14>;
        default: return nullptr;
    }
}

SpectrumK spectrum2_k(int logm) {
    switch (logm) {
        case 12: return &k_spectrum2<12>;
        case 13: return &k_spectrum2<13>;
        case 14: return &k_spectrum2<14>;
        default: return nullptr;
    }
}

PreFftK pre_fft_k(int logn) {
    switch (logn) {
        case 2: return &k_pre_fft<2>;
        case 3: return &k_pre_fft<3>;
        case 4: return &k_pre_fft<4>;
        case 5: return &k_pre_fft<5>;
        case 6: return &k_pre_fft<6>;
        case 7: return &k_pre_fft<7>;
        case 8: return &k_pre_fft<8>;
        case 9: return &k_pre_fft<9>;
        case 10: return &k_pre_fft<10>;
        case 11: return &k_pre_fft<11>;
        case 12: return &k_pre_fft<12>;
        case 13: return &k_pre_fft<13>;
        case 14: return &k_pre_fft<14>;
        default: return nullptr;
    }
}

PreFftK pre_fft2_k(int logm) {
    switch (logm) {
        case 12: return &k_pre_fft2<12>;
        case 13: return &k_pre_fft2<13>;
        case 14: return &k_pre_fft2<14>;
        default: return nullptr;
    }
}

}  // namespace fi
