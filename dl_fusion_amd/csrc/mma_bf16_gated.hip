// Instantiations of the MFMA kernel: dense bf16 GEMM, gated epilogues (SwiGLU, GELU x Mul).
#include "mma_kernel.h"

namespace dlf {

hipError_t launch_mma_bf16_gated(const MmaArgs& a, bool wide, int act, int tile, hipStream_t s) {
    auto go = [&](auto mode_c) -> hipError_t {
        constexpr int M = decltype(mode_c)::value;
        switch (act) {
            case kActSiluMul: return launch_tile<2, M, kActSiluMul, kOutBf16>(a, tile, s);
            case kActGeluMul: return launch_tile<2, M, kActGeluMul, kOutBf16>(a, tile, s);
            case kActGeluErfMul: return launch_tile<2, M, kActGeluErfMul, kOutBf16>(a, tile, s);
            default: return hipErrorInvalidValue;
        }
    };
    return wide ? go(std::integral_constant<int, kDenseWide>{}) : go(std::integral_constant<int, kDense>{});
}

}  // namespace dlf
