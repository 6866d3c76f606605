// Instantiations of the MFMA kernel: dense bf16 GEMM, plain activations.
#include "mma_kernel.h"

namespace dlf {

hipError_t launch_mma_bf16_dense(const MmaArgs& a, bool wide, int act, int tile, hipStream_t s) {
    auto go = [&](auto mode_c) -> hipError_t {
        constexpr int M = decltype(mode_c)::value;
        switch (act) {
            case kActNone: return launch_tile<2, M, kActNone, kOutBf16>(a, tile, s);
            case kActRelu: return launch_tile<2, M, kActRelu, kOutBf16>(a, tile, s);
            case kActGelu: return launch_tile<2, M, kActGelu, kOutBf16>(a, tile, s);
            case kActGeluErf: return launch_tile<2, M, kActGeluErf, kOutBf16>(a, tile, s);
            default: return hipErrorInvalidValue;
        }
    };
    return wide ? go(std::integral_constant<int, kDenseWide>{}) : go(std::integral_constant<int, kDense>{});
}

}  // namespace dlf
