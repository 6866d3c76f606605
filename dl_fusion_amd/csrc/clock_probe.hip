// Shader-clock probe behind the benchmark's clock-derived peak: the matrix pipes' peak rate is
// CUs x shader clock x FLOP per clock per CU, and the clock the chip holds under MFMA load is
// below its 2.4 GHz maximum.  Every workgroup (four waves, one per SIMD) runs four independent
// chains of v_mfma_f32_32x32x16_bf16 back to back and reads the shader clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) before and after; the host
// divides the two differences.
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

__global__ __launch_bounds__(256) void clock_probe_kernel(int iters, uint64_t* stamps) {
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x + e) & 7) * 0.125f);
        b[e] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + e) & 7) * 0.0625f);
    }
    f32x16_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float keep = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) keep += acc[c][e];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        uint64_t* s = stamps + 4 * static_cast<int64_t>(blockIdx.x);
        s[0] = t0;
        s[1] = t1;
        s[2] = r0;
        // a sum that never holds the value below keeps the MFMAs from being removed
        s[3] = keep == -1.0f ? 0 : r1;
    }
}

}  // namespace

hipError_t launch_clock_probe(int workgroups, int iters, uint64_t* stamps, hipStream_t s) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(256), 0, s, iters, stamps);
    return hipGetLastError();
}

}  // namespace dlf
