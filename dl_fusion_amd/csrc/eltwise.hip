// Elementwise kernels of the unfused comparison chain.  Each one reads its
// input(s) from device memory and writes its output back, which is exactly the
// traffic the fused epilogue removes ("OpenPPL算子融合深度解析" §2.1 and §3.3;
// the aitangshan.cn graph-autofusion article counts three HBM round trips for
// MatMul -> BiasAdd -> ReLU).  They stream 16 bytes per lane per step with
// grid-stride loops, so the comparison is against reasonably efficient
// bandwidth-bound passes, not against strawmen.
//
// dt: 0 = fp32, 1 = bf16.  Arithmetic is fp32; bf16 results round to nearest even.
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ float ld(const void* p, int64_t i, int dt) {
    return dt == 0 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
__device__ __forceinline__ void st(void* p, int64_t i, int dt, float v) {
    if (dt == 0)
        static_cast<float*>(p)[i] = v;
    else
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// Vector of 8 values (two 16-byte fp32 loads or one 16-byte bf16 load).
template <int DT>
struct Vec8 {
    float v[8];
    __device__ __forceinline__ void load(const void* p, int64_t i) {
        if constexpr (DT == 0) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
        } else {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float(a[j] << 16);
                v[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
            }
        }
    }
    __device__ __forceinline__ void store(void* p, int64_t i) const {
        if constexpr (DT == 0) {
            f32x4_t a, b;
#pragma unroll
            for (int j = 0; j < 4; ++j) { a[j] = v[j]; b[j] = v[4 + j]; }
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i) = a;
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i + 4) = b;
        } else {
            u32x4_t a;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[j] = static_cast<uint32_t>(f32_to_bf16(v[2 * j])) |
                       (static_cast<uint32_t>(f32_to_bf16(v[2 * j + 1])) << 16);
            *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p) + i) = a;
        }
    }
};

// z = gamma (y - mean) / sqrt(var + eps) + beta per channel, or z = y*scale + shift.
// MODE 0: BatchNorm, MODE 1: scale/shift (scale may be null).
template <int DT, int MODE>
__global__ __launch_bounds__(kBlock) void channel_affine_kernel(int64_t count, int64_t c, const void* y,
                                                                const float* p0, const float* p1,
                                                                const float* p2, const float* p3, float eps,
                                                                void* z) {
    auto f = [&](float v, int64_t ch) -> float {
        if constexpr (MODE == 0)
            return p0[ch] * (v - p2[ch]) / sqrtf(p3[ch] + eps) + p1[ch];
        else
            return p0 ? fmaf(v, p0[ch], p1[ch]) : v + p1[ch];
    };
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    // the channel index advances by a constant per grid-stride step: one division per lane
    if (c % 8 == 0) {
        const int64_t nv = count / 8;
        int64_t ch0 = (8 * t) % c;
        const int64_t dch = (8 * stride) % c;
        for (int64_t v = t; v < nv; v += stride) {
            Vec8<DT> x;
            x.load(y, 8 * v);
#pragma unroll
            for (int j = 0; j < 8; ++j) x.v[j] = f(x.v[j], ch0 + j);
            x.store(z, 8 * v);
            ch0 += dch;
            if (ch0 >= c) ch0 -= c;
        }
    } else {
        int64_t ch = t % c;
        const int64_t dch = stride % c;
        for (int64_t i = t; i < count; i += stride) {
            st(z, i, DT, f(ld(y, i, DT), ch));
            ch += dch;
            if (ch >= c) ch -= c;
        }
    }
}

template <int DT, int OP, int ACT>   // OP 0: add, OP 1: activation
__global__ __launch_bounds__(kBlock) void map_kernel(int64_t count, const void* a, const void* b, void* out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t nv = count / 8;
    for (int64_t v = t; v < nv; v += stride) {
        Vec8<DT> x;
        x.load(a, 8 * v);
        if constexpr (OP == 0) {
            Vec8<DT> y;
            y.load(b, 8 * v);
#pragma unroll
            for (int j = 0; j < 8; ++j) x.v[j] += y.v[j];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) x.v[j] = activate<ACT>(x.v[j]);
        }
        x.store(out, 8 * v);
    }
    for (int64_t i = 8 * nv + t; i < count; i += stride) {
        float v = ld(a, i, DT);
        v = OP == 0 ? v + ld(b, i, DT) : activate<ACT>(v);
        st(out, i, DT, v);
    }
}

__global__ __launch_bounds__(kBlock) void quant_kernel(int64_t count, const float* in, float inv_scale,
                                                       uint8_t* codes) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t nv = count / 4;
    for (int64_t v = t; v < nv; v += stride) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(in + 4 * v);
        reinterpret_cast<uint32_t*>(codes)[v] = quant_e4m3_x4(x[0], x[1], x[2], x[3], inv_scale);
    }
    for (int64_t i = 4 * nv + t; i < count; i += stride)
        codes[i] = static_cast<uint8_t>(quant_e4m3(in[i], inv_scale));
}

unsigned grid_for(int64_t work_items) {
    // enough workgroups to cover the 256 CUs several times over; grid-stride beyond
    int64_t g = (work_items + kBlock - 1) / kBlock;
    if (g > 256 * 16) g = 256 * 16;
    if (g < 1) g = 1;
    return static_cast<unsigned>(g);
}

}  // namespace

hipError_t launch_bn_apply(int64_t rows, int64_t c, int dt, const void* y, const float* gamma,
                           const float* beta, const float* mean, const float* var, float eps, void* z,
                           hipStream_t s) {
    const int64_t count = rows * c;
    if (count == 0) return hipSuccess;
    const unsigned g = grid_for(c % 8 == 0 ? count / 8 : count);
    if (dt == 0)
        hipLaunchKernelGGL((channel_affine_kernel<0, 0>), dim3(g), dim3(kBlock), 0, s, count, c, y, gamma, beta,
                           mean, var, eps, z);
    else
        hipLaunchKernelGGL((channel_affine_kernel<1, 0>), dim3(g), dim3(kBlock), 0, s, count, c, y, gamma, beta,
                           mean, var, eps, z);
    return hipGetLastError();
}

hipError_t launch_scale_shift(int64_t rows, int64_t c, int dt, const void* y, const float* scale,
                              const float* shift, void* z, hipStream_t s) {
    const int64_t count = rows * c;
    if (count == 0) return hipSuccess;
    const unsigned g = grid_for(c % 8 == 0 ? count / 8 : count);
    if (dt == 0)
        hipLaunchKernelGGL((channel_affine_kernel<0, 1>), dim3(g), dim3(kBlock), 0, s, count, c, y, scale, shift,
                           nullptr, nullptr, 0.0f, z);
    else
        hipLaunchKernelGGL((channel_affine_kernel<1, 1>), dim3(g), dim3(kBlock), 0, s, count, c, y, scale, shift,
                           nullptr, nullptr, 0.0f, z);
    return hipGetLastError();
}

hipError_t launch_add(int64_t count, int dt, const void* a, const void* b, void* out, hipStream_t s) {
    if (count == 0) return hipSuccess;
    const unsigned g = grid_for(count / 8 + 1);
    if (dt == 0)
        hipLaunchKernelGGL((map_kernel<0, 0, kActNone>), dim3(g), dim3(kBlock), 0, s, count, a, b, out);
    else
        hipLaunchKernelGGL((map_kernel<1, 0, kActNone>), dim3(g), dim3(kBlock), 0, s, count, a, b, out);
    return hipGetLastError();
}

hipError_t launch_act(int64_t count, int dt, int act, const void* in, void* out, hipStream_t s) {
    if (count == 0) return hipSuccess;
    const unsigned g = grid_for(count / 8 + 1);
#define DLF_ACT_CASE(DT, A) hipLaunchKernelGGL((map_kernel<DT, 1, A>), dim3(g), dim3(kBlock), 0, s, count, in, nullptr, out)
    if (dt == 0) {
        if (act == kActNone) DLF_ACT_CASE(0, kActNone);
        else if (act == kActRelu) DLF_ACT_CASE(0, kActRelu);
        else if (act == kActGelu) DLF_ACT_CASE(0, kActGelu);
        else DLF_ACT_CASE(0, kActGeluErf);
    } else {
        if (act == kActNone) DLF_ACT_CASE(1, kActNone);
        else if (act == kActRelu) DLF_ACT_CASE(1, kActRelu);
        else if (act == kActGelu) DLF_ACT_CASE(1, kActGelu);
        else DLF_ACT_CASE(1, kActGeluErf);
    }
#undef DLF_ACT_CASE
    return hipGetLastError();
}

hipError_t launch_quant(int64_t count, const float* in, float inv_scale, uint8_t* codes, hipStream_t s) {
    if (count == 0) return hipSuccess;
    const unsigned g = grid_for(count / 4 + 1);
    hipLaunchKernelGGL(quant_kernel, dim3(g), dim3(kBlock), 0, s, count, in, inv_scale, codes);
    return hipGetLastError();
}

}  // namespace dlf
