// Instantiations of the MFMA kernel: fp8 GEMM with bf16 output, and the plain fp32 one.
#include "mma_kernel.h"

namespace dlf {

hipError_t launch_mma_fp8_b(const MmaArgs& a, bool wide, int act, int out, int tile, hipStream_t s) {
    auto go = [&](auto mode_c) -> hipError_t {
        constexpr int M = decltype(mode_c)::value;
        if (out == kOutF32) return act == kActNone ? launch_tile<1, M, kActNone, kOutF32>(a, tile, s)
                                                   : hipErrorInvalidValue;
        if (out != kOutBf16) return hipErrorInvalidValue;
        switch (act) {
            case kActNone: return launch_tile<1, M, kActNone, kOutBf16>(a, tile, s);
            case kActRelu: return launch_tile<1, M, kActRelu, kOutBf16>(a, tile, s);
            case kActGelu: return launch_tile<1, M, kActGelu, kOutBf16>(a, tile, s);
            case kActGeluErf: return launch_tile<1, M, kActGeluErf, kOutBf16>(a, tile, s);
            default: return hipErrorInvalidValue;
        }
    };
    return wide ? go(std::integral_constant<int, kDenseWide>{}) : go(std::integral_constant<int, kDense>{});
}

}  // namespace dlf
