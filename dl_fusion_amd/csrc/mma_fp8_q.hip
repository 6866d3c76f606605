// Instantiations of the MFMA kernel: fp8 GEMM with e4m3 output.
#include "mma_kernel.h"

namespace dlf {

hipError_t launch_mma_fp8_q(const MmaArgs& a, bool wide, int act, int tile, hipStream_t s) {
    auto go = [&](auto mode_c) -> hipError_t {
        constexpr int M = decltype(mode_c)::value;
        switch (act) {
            case kActNone: return launch_tile<1, M, kActNone, kOutFp8>(a, tile, s);
            case kActRelu: return launch_tile<1, M, kActRelu, kOutFp8>(a, tile, s);
            case kActGelu: return launch_tile<1, M, kActGelu, kOutFp8>(a, tile, s);
            case kActGeluErf: return launch_tile<1, M, kActGeluErf, kOutFp8>(a, tile, s);
            default: return hipErrorInvalidValue;
        }
    };
    return wide ? go(std::integral_constant<int, kDenseWide>{}) : go(std::integral_constant<int, kDense>{});
}

}  // namespace dlf
