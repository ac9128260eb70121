// FFT gray-block kernels: the one-workgroup transform of every width, the
// two-half class and the split classes (see fi_tables.h).
#include "fi_tables.h"
#include "fi_fft_kernels.h"

namespace fi {

FftTileK fft_tile_k(int logn) {
    switch (logn) {
        case 2: return &k_fft_tile<2>;
        case 3: return &k_fft_tile<3>;
        case 4: return &k_fft_tile<4>;
        case 5: return &k_fft_tile<5>;
        case 6: return &k_fft_tile<6>;
        case 7: return &k_fft_tile<7>;
        case 8: return &k_fft_tile<8>;
        case 9: return &k_fft_tile<9>;
        case 10: return &k_fft_tile<10>;
        case 11: return &k_fft_tile<11>;
        case 12: return &k_fft_tile<12>;
        case 13: return &k_fft_tile<13>;
        case 14: return &k_fft_tile<14>;
        default: return nullptr;
    }
}

FftTileK fft_tile2_k(int logm) {
    switch (logm) {
        case 12: return &k_fft_tile2<12>;
        case 13: return &k_fft_tile2<13>;
        case 14: return &k_fft_tile2<14>;
        default: return nullptr;
    }
}

SubFwdK sub_fwd_k(int logv) {
    switch (logv) {
        case 12: return &k_fft_sub_fwd<12>;
        case 13: return &k_fft_sub_fwd<13>;
        case 14: return &k_fft_sub_fwd<14>;
        default: return nullptr;
    }
}

template <int LOGV>
SubInvK sub_inv_kk(int K) {
    switch (K) {
        case 4: return &k_fft_sub_inv<LOGV, 4>;
        case 8: return &k_fft_sub_inv<LOGV, 8>;
        default: return &k_fft_sub_inv<LOGV, 0>;
    }
}

SubInvK sub_inv_k(int logv, int K) {
    switch (logv) {
        case 12: return sub_inv_kk<12>(K);
        case 13: return sub_inv_kk<13>(K);
        case 14: return sub_inv_kk<14>(K);
        default: return nullptr;
    }
}

}  // namespace fi
