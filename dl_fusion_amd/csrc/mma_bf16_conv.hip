// Instantiations of the MFMA kernel: bf16 implicit-GEMM convolution.
#include "mma_kernel.h"

namespace dlf {

hipError_t launch_mma_bf16_conv(const MmaArgs& a, int act, int tile, hipStream_t s) {
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
    // a 64-byte slice (32 bf16) stays inside one kernel tap when Cin % 32 == 0
    if (a.Cin % 32 == 0) return go(std::integral_constant<int, kConvAligned>{});
    // a 16-byte chunk (8 bf16) stays inside one tap when Cin % 8 == 0; otherwise value by value
    if (a.Cin % 8 == 0) return go(std::integral_constant<int, kConvGeneric>{});
    return go(std::integral_constant<int, kConvAnyC>{});
}

}  // namespace dlf
