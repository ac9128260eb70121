// Hyena-style block kernels, one variant per batch size (see fi_tables.h).
#include "fi_tables.h"
#include "fi_block.h"

namespace fi {

namespace {
template <int B>
struct BlockKernels {
    static constexpr HyProjK proj = &k_hy_proj<B>;
    static constexpr HyStepK up = &k_hy_up<B>;
    static constexpr HyStepK down = &k_hy_down<B>;
};
}  // namespace

HyProjK hy_proj_k(int B) {
    switch (B) {
        case 1: return BlockKernels<1>::proj;
        case 2: return BlockKernels<2>::proj;
        case 3: return BlockKernels<3>::proj;
        case 4: return BlockKernels<4>::proj;
        case 5: return BlockKernels<5>::proj;
        case 6: return BlockKernels<6>::proj;
        case 7: return BlockKernels<7>::proj;
        case 8: return BlockKernels<8>::proj;
        default: return nullptr;
    }
}

HyStepK hy_up_k(int B) {
    switch (B) {
        case 1: return BlockKernels<1>::up;
        case 2: return BlockKernels<2>::up;
        case 3: return BlockKernels<3>::up;
        case 4: return BlockKernels<4>::up;
        case 5: return BlockKernels<5>::up;
        case 6: return BlockKernels<6>::up;
        case 7: return BlockKernels<7>::up;
        case 8: return BlockKernels<8>::up;
        default: return nullptr;
    }
}

HyStepK hy_down_k(int B) {
    switch (B) {
        case 1: return BlockKernels<1>::down;
        case 2: return BlockKernels<2>::down;
        case 3: return BlockKernels<3>::down;
        case 4: return BlockKernels<4>::down;
        case 5: return BlockKernels<5>::down;
        case 6: return BlockKernels<6>::down;
        case 7: return BlockKernels<7>::down;
        case 8: return BlockKernels<8>::down;
        default: return nullptr;
    }
}

}  // namespace fi
