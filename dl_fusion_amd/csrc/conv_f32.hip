// fp32 direct convolution with the register epilogue (bias -> residual -> act).
//
// Used for fp32 layers (small, latency-bound shapes).  A workgroup computes a
// tile of 64 output pixels x TC output channels.  The K dimension
// (k = (r*KW + s)*Cin + ci) is walked in slices of 64: each slice of the
// weights is staged in LDS transposed to [k][channel] (consecutive lanes read
// consecutive channels), and the matching im2col slice of the input (64 pixels
// x 64 k, zero outside the image) is staged as [pixel][k] and read as a
// broadcast.  Each lane accumulates 64*TC/256 outputs in fp32 and applies the
// epilogue of "OpenPPL算子融合深度解析" §4.3 before its single store.
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

constexpr int kPix = 64;     // output pixels per workgroup
constexpr int kKs = 64;      // K slice

template <int TC, int ACT>
__global__ __launch_bounds__(256) void conv_f32_kernel(const ConvF32Args p) {
    constexpr int PG = 256 / TC;            // pixel groups
    constexpr int PPT = kPix / PG;          // pixels per lane
    __shared__ float ws[kKs][TC + 1];
    __shared__ float xs[kPix][kKs + 1];

    const int tid = static_cast<int>(threadIdx.x);
    const int co_l = tid % TC, pg = tid / TC;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPix;
    const int c0 = static_cast<int>(blockIdx.y) * TC;
    const int co = c0 + co_l;

    float acc[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) acc[j] = 0.0f;

    const int hw = p.Ho * p.Wo;
    for (int k0 = 0; k0 < p.K; k0 += kKs) {
        // weights slice -> ws[k][channel]
        for (int e = tid; e < kKs * TC; e += 256) {
            const int c = e / kKs, k = e % kKs;
            const int gc = c0 + c, gk = k0 + k;
            ws[k][c] = (gc < p.Cout && gk < p.K) ? p.w[static_cast<int64_t>(gc) * p.K + gk] : 0.0f;
        }
        // im2col slice -> xs[pixel][k]
        for (int e = tid; e < kPix * kKs; e += 256) {
            const int pix = e / kKs, k = e % kKs;
            const int64_t m = p0 + pix;
            const int gk = k0 + k;
            float v = 0.0f;
            if (m < p.M && gk < p.K) {
                const int tap = gk / p.Cin, ci = gk - tap * p.Cin;
                const int r = tap / p.KW, s = tap - r * p.KW;
                const int img = static_cast<int>(m / hw), rem = static_cast<int>(m % hw);
                const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
                const int hi = ho * p.SH - p.PH + r, wi = wo * p.SW - p.PW + s;
                if (hi >= 0 && hi < p.H && wi >= 0 && wi < p.W)
                    v = p.x[((static_cast<int64_t>(img) * p.H + hi) * p.W + wi) * p.Cin + ci];
            }
            xs[pix][k] = v;
        }
        __syncthreads();
        const int kn = min(kKs, p.K - k0);
        for (int k = 0; k < kn; ++k) {
            const float wv = ws[k][co_l];
#pragma unroll
            for (int j = 0; j < PPT; ++j) acc[j] = fmaf(xs[pg + PG * j][k], wv, acc[j]);
        }
        __syncthreads();
    }

    if (co >= p.Cout) return;
    const float b = p.bias ? p.bias[co] : 0.0f;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int64_t m = p0 + pg + PG * j;
        if (m >= p.M) continue;
        const int64_t idx = m * p.Cout + co;
        float v = acc[j] + b;
        if (p.res) v += p.res[idx];
        p.y[idx] = activate<ACT>(v);
    }
}

template <int TC>
hipError_t launch_tc(const ConvF32Args& a, int act, hipStream_t s) {
    const int64_t gx = (a.M + kPix - 1) / kPix;
    const int gy = (a.Cout + TC - 1) / TC;
    if (gx == 0 || gy == 0) return hipSuccess;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
    switch (act) {
        case kActNone: hipLaunchKernelGGL((conv_f32_kernel<TC, kActNone>), grid, dim3(256), 0, s, a); break;
        case kActRelu: hipLaunchKernelGGL((conv_f32_kernel<TC, kActRelu>), grid, dim3(256), 0, s, a); break;
        case kActGelu: hipLaunchKernelGGL((conv_f32_kernel<TC, kActGelu>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_f32(const ConvF32Args& a, int act, hipStream_t s) {
    return a.Cout <= 32 ? launch_tc<32>(a, act, s) : launch_tc<64>(a, act, s);
}

}  // namespace dlf
