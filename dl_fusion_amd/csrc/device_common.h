// Device-side building blocks shared by the HIP kernels of libdlfusion:
// vector types for the gfx950 MFMA builtins, bf16 conversion, the epilogue
// activations and the e4m3 output quantiser.
//
// Epilogue order and activation numbering follow the conv epilogue of
// "OpenPPL算子融合深度解析" §4.3 (bias, then residual, then activation
// 0 none / 1 ReLU / 2 GELU-tanh, applied to the accumulator before the one
// store); the quantiser is the static-scale FP8 store of
// "FlashRT 跨层融合深度解析" §3 with the clamp a quantised ReLU needs
// ("OpenPPL算子融合深度解析" §6.4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum : int { kActNone = 0, kActRelu = 1, kActGelu = 2, kActGeluErf = 3 };
// gated epilogues: the GEMM's columns come in (gate, up) pairs and the output is gate_act(g) * u
enum : int { kActSiluMul = 4, kActGeluMul = 5, kActGeluErfMul = 6 };
enum : int { kOutBf16 = 0, kOutFp8 = 1, kOutF32 = 2 };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// GELU, tanh form: 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3).
// Evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), i.e.
// gelu(v) = v / (1 + 2^(-2 u log2 e)), with the hardware exp2 and reciprocal
// (about 1 ulp each).  This form has no cancellation for negative v and gives
// -0 / v in the saturated tails.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float k = -2.0f * 0.797884560802865355879892f * 1.442695040888963407359924f;  // -2 sqrt(2/pi) log2(e)
    const float t = v * fmaf(0.044715f * v, v, 1.0f);                                   // v + 0.044715 v^3
    const float e = __builtin_amdgcn_exp2f(k * t);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// GELU, exact form: v Phi(v) = 0.5 v erfc(-z), z = v / sqrt(2).  erfc(|z|) is the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erfc(x) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2), t = 1 / (1 + p x), x >= 0,
// absolute error <= 1.5e-7; erfc(-|z|) = 2 - erfc(|z|).  About 15 instructions against ~40
// for the library erfc, and far below the bf16 rounding of the result.
__device__ __forceinline__ float gelu_erf(float v) {
    const float z = 0.70710678118654752440f * v;
    const float az = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, az, 1.0f));
    const float poly =
        t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
                 0.254829592f);
    const float e = poly * __builtin_amdgcn_exp2f(-1.44269504088896340736f * az * az);   // erfc(|z|)
    return 0.5f * v * (z >= 0.0f ? 2.0f - e : e);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

// Two values rounded to bf16 (nearest even) in one conversion; a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// ReLU of two packed bf16 values: a value with the sign bit set becomes +0 (as a signed
// 16-bit integer it is negative, so one packed integer max with 0 does both halves).
// Rounding to nearest keeps the sign, so ReLU after the rounding equals the rounding of ReLU.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t u) {
    const i16x2_t s = __builtin_bit_cast(i16x2_t, u);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(s, i16x2_t{0, 0}));
}

// SiLU, v / (1 + e^-v), with the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896340736f * v));
}

// The gate activation of a gated epilogue.
template <int ACT>
__device__ __forceinline__ float gate_act(float g) {
    if constexpr (ACT == kActSiluMul) {
        return silu(g);
    } else if constexpr (ACT == kActGeluMul) {
        return gelu_tanh(g);
    } else {
        static_assert(ACT == kActGeluErfMul, "gated epilogue");
        return gelu_erf(g);
    }
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
    if constexpr (ACT == kActRelu) {
        return v > 0.0f ? v : 0.0f;
    } else if constexpr (ACT == kActGelu) {
        return gelu_tanh(v);
    } else if constexpr (ACT == kActGeluErf) {
        return gelu_erf(v);
    } else {
        return v;
    }
}

// Static e4m3 quantisation: code = Q(fp32(v * inv_scale)).  The product is one
// IEEE fp32 multiply (never contracted into a neighbouring add), clamped to the
// largest finite e4m3 magnitude 448, then converted by the hardware's OCP e4m3
// conversion (round to nearest even).
__device__ __forceinline__ uint32_t quant_e4m3(float v, float inv_scale) {
    float p = __fmul_rn(v, inv_scale);
    p = fminf(fmaxf(p, -448.0f), 448.0f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(p, p, 0, false)) & 0xFFu;
}

// Four codes packed little-endian into one 32-bit word.
__device__ __forceinline__ uint32_t quant_e4m3_x4(float a, float b, float c, float d, float inv_scale) {
    float pa = fminf(fmaxf(__fmul_rn(a, inv_scale), -448.0f), 448.0f);
    float pb = fminf(fmaxf(__fmul_rn(b, inv_scale), -448.0f), 448.0f);
    float pc = fminf(fmaxf(__fmul_rn(c, inv_scale), -448.0f), 448.0f);
    float pd = fminf(fmaxf(__fmul_rn(d, inv_scale), -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(pa, pb, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(pc, pd, w, true);
    return static_cast<uint32_t>(w);
}

}  // namespace dlf
