// Dispatch of the MFMA GEMM / implicit-GEMM kernel (mma_kernel.h) to its instantiation groups
// (mma_bf16_dense.hip, mma_bf16_gated.hip, mma_bf16_conv.hip, mma_fp8_q.hip, mma_fp8_b.hip).
#include "device_common.h"
#include "kernels.h"

namespace dlf {

int mma_tile_rows(int tile) {
    switch (tile) {
        case kTile256x256: return 256;
        case kTile128x128: case kTile128x64: return 128;
        case kTile64x64: return 64;
        default: return 0;
    }
}

int mma_tile_cols(int tile) {
    switch (tile) {
        case kTile256x256: return 256;
        case kTile128x128: return 128;
        default: return 64;
    }
}

namespace {

// The buffer form holds while a 256-row panel spans less than 2 GB (rows under 8 MB); longer
// rows take the global-address form.
bool dense_buffer_ok(const MmaArgs& a, int elem) { return static_cast<int64_t>(a.K) * elem < (int64_t(1) << 23); }

}  // namespace

hipError_t launch_mma_bf16(const MmaArgs& a, bool conv, int act, int tile, hipStream_t s) {
    if (conv) return launch_mma_bf16_conv(a, act, tile, s);
    const bool wide = !dense_buffer_ok(a, 2);
    if (act >= kActSiluMul) return launch_mma_bf16_gated(a, wide, act, tile, s);
    return launch_mma_bf16_dense(a, wide, act, tile, s);
}

hipError_t launch_mma_fp8(const MmaArgs& a, int act, int out, int tile, hipStream_t s) {
    const bool wide = !dense_buffer_ok(a, 1);
    if (out == kOutFp8) return launch_mma_fp8_q(a, wide, act, tile, s);
    return launch_mma_fp8_b(a, wide, act, out, tile, s);
}

}  // namespace dlf
