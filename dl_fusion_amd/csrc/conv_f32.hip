// fp32 direct convolution with the register epilogue (bias -> residual -> act).
//
// Used for fp32 layers (small, latency-bound shapes: a 1x32x32 16->32 3x3 layer is 9.4 MFLOP,
// a few hundred cycles of FMA work spread over the chip, so its time is launch, one memory
// round trip and the store).  Each lane computes one output element (pixel m, channel co);
// a workgroup covers 256/TC pixels x TC channels.
//
// conv_f32_regw_kernel (K <= 256, Cin a multiple of 4): one pass, 32 x PPB lanes.  The workgroup
// copies its 32 channels' K weights into LDS once (16-byte loads of one contiguous block) while
// it gathers the receptive fields of its pixels (one 16-byte load per tap and 4 channels, zero
// outside the image), every load of both issued before the first LDS store; after one barrier a lane reads 4 weights of its channel and 4 input values
// of its pixel per pair of LDS reads (the lanes of a pixel read the same input address) for 4
// FMAs, sixteen pairs of reads in flight at a time (the rows are zero-padded to whole groups).
//
// conv_f32_kernel (any other shape): weights staged in LDS transposed to [k][channel] in
// slices of 4096 values, together with the im2col rows of its pixels, each gathered by
// independent loads so that a slice costs one memory round trip.
//
// fp32 accumulation, then the epilogue of "OpenPPL算子融合深度解析" §4.3 before the single store.
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

template <int TC, int ACT>
__global__ __launch_bounds__(256) void conv_f32_kernel(const ConvF32Args p) {
    constexpr int PPB = 256 / TC;         // pixels per workgroup
    constexpr int KS = 4096 / TC;         // K values per slice (16 KB of weights in LDS)
    __shared__ float ws[KS][TC];
    __shared__ float xs[PPB][KS + 1];

    const int tid = static_cast<int>(threadIdx.x);
    const int co_l = tid % TC, pl = tid / TC;
    const int m0 = static_cast<int>(blockIdx.x) * PPB;   // M <= 2^30 (checked on the host)
    const int c0 = static_cast<int>(blockIdx.y) * TC;
    const int co = c0 + co_l;
    const int hw = p.Ho * p.Wo;

    // the epilogue's bias and residual are loaded before the K loop, not after it
    const int m = m0 + pl;
    const bool live = m < p.M && co < p.Cout;
    const int64_t idx = static_cast<int64_t>(m) * p.Cout + co;
    const float bco = p.bias && co < p.Cout ? p.bias[co] : 0.0f;
    const float rv = p.res && live ? p.res[idx] : 0.0f;
    float acc = 0.0f;
    for (int k0 = 0; k0 < p.K; k0 += KS) {
        // weights slice -> ws[k][channel]; consecutive lanes read consecutive k
        for (int e = tid; e < KS * TC; e += 256) {
            const int c = e / KS, kk = e - c * KS;
            const int gc = c0 + c, gk = k0 + kk;
            ws[kk][c] = (gc < p.Cout && gk < p.K) ? p.w[static_cast<int64_t>(gc) * p.K + gk] : 0.0f;
        }
        // im2col rows of this workgroup's pixels -> xs[pixel][k]; every load is independent
        for (int e = tid; e < PPB * KS; e += 256) {
            const int q = e / KS, kk = e - q * KS;
            const int mq = m0 + q, gk = k0 + kk;
            float v = 0.0f;
            if (mq < p.M && gk < p.K) {
                const int img = mq / hw, rem = mq - img * hw;
                const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
                const int tap = gk / p.Cin, ci = gk - tap * p.Cin;
                const int r = tap / p.KW, s = tap - r * p.KW;
                const int hi = ho * p.SH - p.PH + r, wi = wo * p.SW - p.PW + s;
                if (static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                    static_cast<unsigned>(wi) < static_cast<unsigned>(p.W))
                    v = p.x[((static_cast<int64_t>(img) * p.H + hi) * p.W + wi) * p.Cin + ci];
            }
            xs[q][kk] = v;
        }
        __syncthreads();
        const int kn = min(KS, p.K - k0);
#pragma unroll 8
        for (int kk = 0; kk < kn; ++kk) acc = fmaf(xs[pl][kk], ws[kk][co_l], acc);
        __syncthreads();
    }

    if (!live) return;
    float v = acc + bco;
    if (p.res) v += rv;
    p.y[idx] = activate<ACT>(v);
}

// K <= KMAX (a multiple of 4), Cin % 4 == 0.  32 PPB lanes: PPB pixels x 32 channels.
template <int KMAX, int PPB, int ACT>
__global__ __launch_bounds__(32 * PPB) void conv_f32_regw_kernel(const ConvF32Args p) {
    constexpr int TC = 32, K4 = KMAX / 4, NT = 32 * PPB;
    // weight rows padded by 16 bytes: the 16 channels one 16-byte LDS read serves per cycle then
    // start in 16 distinct 4-bank groups (row stride KMAX + 4 words, a multiple of 4 that is not
    // a multiple of 64 for KMAX = 64, 160, 256)
    constexpr int WS = KMAX + 4;
    __shared__ f32x4_t ws[TC * WS / 4];
    __shared__ f32x4_t xs[PPB][K4];
    const int tid = static_cast<int>(threadIdx.x);
    const int co_l = tid % TC, pl = tid / TC;
    const int m0 = static_cast<int>(blockIdx.x) * PPB;
    const int c0 = static_cast<int>(blockIdx.y) * TC;
    const int co = c0 + co_l;
    const int k4n = p.K >> 2;
    // Every global load of both copies below is issued before the first LDS store, so the staging
    // costs one memory round trip instead of one per loop trip.  The workgroup's weight rows
    // c0 .. c0 + 31 are one block of 32 K values (K % 4 == 0, w 16-byte aligned); rows past Cout
    // are left unread and their results never stored.
    const int rows = min(TC, p.Cout - c0);
    const f32x4_t* const wblk = reinterpret_cast<const f32x4_t*>(p.w + static_cast<int64_t>(c0) * p.K);
    constexpr int WIT = (TC * K4 + NT - 1) / NT, XIT = (PPB * K4 + NT - 1) / NT;
    f32x4_t wstage[WIT], xstage[XIT];
#pragma unroll
    for (int i = 0; i < WIT; ++i) {
        const int e = tid + i * NT;
        if (e < rows * k4n) wstage[i] = wblk[e];
    }
    // receptive fields of the workgroup's pixels: item e = (pixel, 4 consecutive k), one tap each
    const int hw = p.Ho * p.Wo;
    const int c4 = p.Cin >> 2;
#pragma unroll
    for (int i = 0; i < XIT; ++i) {
        const int e = tid + i * NT;
        xstage[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int q = e / k4n, kk4 = e - q * k4n;
        const int m = m0 + q;
        if (e < PPB * k4n && m < p.M) {
            const int img = m / hw, rem = m - img * hw;
            const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
            const int tap = kk4 / c4, ci = (kk4 - tap * c4) * 4;
            const int r = tap / p.KW, sx = tap - r * p.KW;
            const int hi = ho * p.SH - p.PH + r, wi = wo * p.SW - p.PW + sx;
            if (static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                static_cast<unsigned>(wi) < static_cast<unsigned>(p.W))
                xstage[i] = *reinterpret_cast<const f32x4_t*>(
                    p.x + ((static_cast<int64_t>(img) * p.H + hi) * p.W + wi) * p.Cin + ci);
        }
    }
    // the epilogue's bias and residual go out with the staging loads: loaded after the
    // contraction, they would add a memory round trip to the end of the kernel
    const int m = m0 + pl;
    const bool live = m < p.M && co < p.Cout;
    const int64_t idx = static_cast<int64_t>(m) * p.Cout + co;
    const float bco = p.bias && co < p.Cout ? p.bias[co] : 0.0f;
    const float rv = p.res && live ? p.res[idx] : 0.0f;
#pragma unroll
    for (int i = 0; i < WIT; ++i) {
        const int e = tid + i * NT;
        if (e < rows * k4n) {
            const int r = e / k4n, q = e - r * k4n;
            ws[r * (WS / 4) + q] = wstage[i];
        }
    }
#pragma unroll
    for (int i = 0; i < XIT; ++i) {
        const int e = tid + i * NT;
        if (e < PPB * k4n) {
            const int q = e / k4n, kk4 = e - q * k4n;
            xs[q][kk4] = xstage[i];
        }
    }
    // zeros past K in every weight and pixel row: the contraction below then runs whole groups
    // of chunks, with one guard per group instead of one per chunk
    const int kt4 = K4 - k4n;
    for (int e = tid; e < (TC + PPB) * kt4; e += NT) {
        const int r = e / kt4, q = k4n + (e - r * kt4);
        if (r < TC)
            ws[r * (WS / 4) + q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        else
            xs[r - TC][q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __syncthreads();
    if (!live) return;
    const f32x4_t* const wrow = ws + co_l * (WS / 4);
    float acc0 = 0.0f, acc1 = 0.0f;    // two chains: even and odd k
    // groups of 16 chunks, each its own basic block: a group's 32 LDS reads go out together, then
    // its 64 FMAs.  With a guard per chunk every pair of reads waited out its own LDS round trip;
    // with no guard at all the compiler kept the whole row's reads in registers and spilled.
    constexpr int GQ = 16;
#pragma unroll
    for (int q0 = 0; q0 < K4; q0 += GQ) {
        if (q0 < k4n) {
            f32x4_t xq[GQ], wq[GQ];
#pragma unroll
            for (int u = 0; u < GQ && q0 + u < K4; ++u) {
                xq[u] = xs[pl][q0 + u];
                wq[u] = wrow[q0 + u];
            }
#pragma unroll
            for (int u = 0; u < GQ && q0 + u < K4; ++u) {
                acc0 = fmaf(xq[u][0], wq[u][0], acc0);
                acc1 = fmaf(xq[u][1], wq[u][1], acc1);
                acc0 = fmaf(xq[u][2], wq[u][2], acc0);
                acc1 = fmaf(xq[u][3], wq[u][3], acc1);
            }
        }
    }
    float v = (acc0 + acc1) + bco;
    if (p.res) v += rv;
    p.y[idx] = activate<ACT>(v);
}

template <int KMAX, int PPB>
hipError_t launch_regw_ppb(const ConvF32Args& a, int act, hipStream_t s) {
    const int64_t gx = (a.M + PPB - 1) / PPB;
    const int gy = (a.Cout + 31) / 32;
    if (gx == 0 || gy == 0) return hipSuccess;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), block(32 * PPB);
    switch (act) {
        case kActNone: hipLaunchKernelGGL((conv_f32_regw_kernel<KMAX, PPB, kActNone>), grid, block, 0, s, a); break;
        case kActRelu: hipLaunchKernelGGL((conv_f32_regw_kernel<KMAX, PPB, kActRelu>), grid, block, 0, s, a); break;
        case kActGelu: hipLaunchKernelGGL((conv_f32_regw_kernel<KMAX, PPB, kActGelu>), grid, block, 0, s, a); break;
        case kActGeluErf:
            hipLaunchKernelGGL((conv_f32_regw_kernel<KMAX, PPB, kActGeluErf>), grid, block, 0, s, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The weights are staged once per workgroup, so larger pixel blocks cut the weight traffic: 16
// pixels a workgroup measured best on a 1x32x32 16->32 layer (64 workgroups, 4.0 us a launch in
// a graph; 4.29 us against 5.2 us with 8 before the contraction read its operands in groups; before
// the staging loads were all issued up front, 4.45 us with 16, 4.7 us with 8, 5.1 us with 4 and
// 5.4 us with 32).  Smaller blocks only where 16 would leave
// fewer than 64 workgroups.
template <int KMAX>
hipError_t launch_regw(const ConvF32Args& a, int act, hipStream_t s) {
    const int64_t cb = (a.Cout + 31) / 32;
    auto wgs = [&](int ppb) { return (static_cast<int64_t>(a.M) + ppb - 1) / ppb * cb; };
    if (wgs(16) >= 64) return launch_regw_ppb<KMAX, 16>(a, act, s);
    if (wgs(8) >= 64) return launch_regw_ppb<KMAX, 8>(a, act, s);
    if (wgs(4) >= 64) return launch_regw_ppb<KMAX, 4>(a, act, s);
    return launch_regw_ppb<KMAX, 2>(a, act, s);
}

template <int TC>
hipError_t launch_tc(const ConvF32Args& a, int act, hipStream_t s) {
    constexpr int PPB = 256 / TC;
    const int64_t gx = (a.M + PPB - 1) / PPB;
    const int gy = (a.Cout + TC - 1) / TC;
    if (gx == 0 || gy == 0) return hipSuccess;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
    switch (act) {
        case kActNone: hipLaunchKernelGGL((conv_f32_kernel<TC, kActNone>), grid, dim3(256), 0, s, a); break;
        case kActRelu: hipLaunchKernelGGL((conv_f32_kernel<TC, kActRelu>), grid, dim3(256), 0, s, a); break;
        case kActGelu: hipLaunchKernelGGL((conv_f32_kernel<TC, kActGelu>), grid, dim3(256), 0, s, a); break;
        case kActGeluErf: hipLaunchKernelGGL((conv_f32_kernel<TC, kActGeluErf>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_f32(const ConvF32Args& a, int act, hipStream_t s) {
    // the register path wants 16-byte rows of x and w (Cin % 4 == 0) and K <= 256; x, w, y are
    // 16-byte aligned (checked on the host)
    if (a.Cin % 4 == 0 && a.K > 0 && a.K <= 256) {
        if (a.K <= 64) return launch_regw<64>(a, act, s);
        if (a.K <= 160) return launch_regw<160>(a, act, s);
        return launch_regw<256>(a, act, s);
    }
    return a.Cout <= 32 ? launch_tc<32>(a, act, s) : launch_tc<64>(a, act, s);
}

}  // namespace dlf
