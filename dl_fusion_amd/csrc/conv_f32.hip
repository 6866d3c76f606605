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
    constexpr int PPT = kPix / PG;          // output pixels per lane
    constexpr int XS = kPix * kKs / 256;    // im2col entries each lane stages per slice
    __shared__ float ws[kKs][TC + 1];
    __shared__ float xs[kPix][kKs + 1];

    const int tid = static_cast<int>(threadIdx.x);
    const int co_l = tid % TC, pg = tid / TC;
    const int p0 = static_cast<int>(blockIdx.x) * kPix;   // M <= 2^30 (checked on the host)
    const int c0 = static_cast<int>(blockIdx.y) * TC;
    const int co = c0 + co_l;

    // staging assignment: this lane stages column kq of the slice for pixels kp + 4 i
    const int kq = tid & (kKs - 1), kp = tid >> 6;
    int px_base[XS], px_h[XS], px_w[XS];
    const int hw = p.Ho * p.Wo;
#pragma unroll
    for (int i = 0; i < XS; ++i) {
        const int m = p0 + kp + 4 * i;
        const int mm = m < p.M ? m : 0;
        const int img = mm / hw, rem = mm - img * hw;
        const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
        const int h0 = ho * p.SH - p.PH;
        px_w[i] = wo * p.SW - p.PW;
        px_base[i] = (img * p.H + h0) * p.W + px_w[i];
        px_h[i] = m < p.M ? h0 : -(1 << 29);   // rows past M never pass the bounds test
    }

    float acc[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) acc[j] = 0.0f;

    for (int k0 = 0; k0 < p.K; k0 += kKs) {
        const int gk = k0 + kq;
        const bool k_ok = gk < p.K;
        // weights slice -> ws[k][channel]
#pragma unroll
        for (int i = 0; i < kKs * TC / 256; ++i) {
            const int c = kp + 4 * i;
            const int gc = c0 + c;
            ws[kq][c] = (gc < p.Cout && k_ok) ? p.w[static_cast<int64_t>(gc) * p.K + gk] : 0.0f;
        }
        // im2col slice -> xs[pixel][k]: one (tap, ci) decomposition per lane per slice
        int r = 0, s = 0, ci = 0;
        if (k_ok) {
            const int tap = gk / p.Cin;
            ci = gk - tap * p.Cin;
            r = tap / p.KW;
            s = tap - r * p.KW;
        }
#pragma unroll
        for (int i = 0; i < XS; ++i) {
            const int hi = px_h[i] + r, wi = px_w[i] + s;
            float v = 0.0f;
            if (k_ok && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                static_cast<unsigned>(wi) < static_cast<unsigned>(p.W))
                v = p.x[static_cast<int64_t>(px_base[i] + r * p.W + s) * p.Cin + ci];
            xs[kp + 4 * i][kq] = v;
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
        const int m = p0 + pg + PG * j;
        if (m >= p.M) continue;
        const int64_t idx = static_cast<int64_t>(m) * p.Cout + co;
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
