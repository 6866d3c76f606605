// bf16 convolution for images with few channels (c_in <= 4, such as the 3-channel input of
// a ResNet stem: 7x7, stride 2, pad 3) with the register epilogue of the fused operator
// (bias -> residual -> activation -> one rounding, each output element stored once; the
// conv epilogue of "OpenPPL算子融合深度解析" §4.3 with the folded BN of §3.1).
//
// A 16-byte-chunk implicit GEMM wastes most of its loads here: a chunk of 8 k-values spans
// several taps and is not aligned.  Instead each workgroup keeps in LDS
//   - its 64 output channels' weights, re-laid as [co][r][s (KW rounded up to 4)][4 channels],
//   - the input patch under `th` output rows, as [row][column][4 channels] (8 bytes a pixel,
//     zero outside the image and in the fourth channel),
// so that one lane's 8 k-values of a 32x32x16 MFMA (two neighbouring taps s, s+1 of one
// kernel row, four channels each) are 16 contiguous bytes for both operands.  Both are
// filled with 16-byte global loads of whole input rows and of the weight block (the host
// checks that rows and the block are multiples of 16 bytes) and scattered value by value
// into the padded layouts.  The K loop then runs KH x ceil(KW/4) MFMA steps per 32-pixel
// fragment and channel fragment, out of LDS only.
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

constexpr int kSmallLds = 65536;   // bytes: weights first, then the patch
constexpr int kSmallStage = 4096;  // bytes a wave: one finished 32-pixel fragment

// bytes between two output channels' weights: KH kwp 8, plus 16 where that is an even number
// of 16-byte chunks, so that the 32 lanes' fragment reads (one channel each) fall in distinct
// LDS banks
__host__ __device__ inline int smallc_wstride(int kh, int kwp) {
    const int b = kh * kwp * 8;
    return (b / 16) % 2 == 0 ? b + 16 : b;
}

template <int ACT, bool RES>
__global__ __launch_bounds__(256, 2) void conv_smallc_kernel(const SmallCArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmallLds + 4 * kSmallStage];
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    int bid = static_cast<int>(blockIdx.x);
    const int cblk = bid % p.co_blocks;
    bid /= p.co_blocks;
    const int rt = bid % p.row_tiles;
    const int img = bid / p.row_tiles;
    const int co0 = cblk * 64;
    const int nco = min(64, p.Cout - co0);                  // 32 or 64
    const int ho0 = rt * p.th;
    const int rows = min(p.th, p.Ho - ho0);
    const int wstride = smallc_wstride(p.KH, p.kwp);
    uint8_t* const sw = smem;
    uint8_t* const sx = smem + 64 * wstride;

    // ---- zero both regions (padding taps, the fourth channel, rows and columns outside) ----
    for (int i = tid; i < kSmallLds / 16; i += 256)
        *reinterpret_cast<u32x4_t*>(smem + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    // ---- weights of channels co0 .. co0+nco-1: one contiguous block of nco*K values.  Four
    //      16-byte loads per lane go out before their values are scattered; the (co, r, s, ci)
    //      position of a chunk's first value is divided out once, the next seven step on. ----
    const int K = p.KH * p.KW * p.Cin;
    {
        const uint8_t* const src = reinterpret_cast<const uint8_t*>(p.w) + static_cast<int64_t>(co0) * K * 2;
        const int chunks = nco * K / 8;                     // whole: nco % 8 == 0
        for (int c0 = tid; c0 < chunks; c0 += 4 * 256) {
            u32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (c0 + 256 * u < chunks) v[u] = *reinterpret_cast<const u32x4_t*>(src + 16 * (c0 + 256 * u));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + 256 * u;
                if (c >= chunks) break;
                const int idx = 8 * c;
                int co = idx / K, k = idx - co * K;
                int r = k / (p.KW * p.Cin), rem = k - r * p.KW * p.Cin;
                int sx_ = rem / p.Cin, ci = rem - sx_ * p.Cin;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t word = v[u][e >> 1];
                    const uint16_t val = static_cast<uint16_t>((e & 1) ? (word >> 16) : (word & 0xFFFFu));
                    *reinterpret_cast<uint16_t*>(sw + co * wstride + ((r * p.kwp + sx_) * 4 + ci) * 2) = val;
                    if (++ci == p.Cin) {
                        ci = 0;
                        if (++sx_ == p.KW) {
                            sx_ = 0;
                            if (++r == p.KH) {
                                r = 0;
                                ++co;
                            }
                        }
                    }
                }
            }
        }
    }
    // ---- input rows hi0 .. hi0+prows-1 of this image, whole rows (W*Cin values each), four
    //      loads per lane in flight as above ----
    const int hi0 = ho0 * p.SH - p.PH;
    const int prows = (rows - 1) * p.SH + p.KH;
    const int row_vals = p.W * p.Cin;
    const int row_chunks = row_vals / 8;                   // whole: the host checks W*Cin % 8 == 0
    {
        const uint8_t* const xb = reinterpret_cast<const uint8_t*>(p.x) + static_cast<int64_t>(img) * p.H * row_vals * 2;
        const int total = prows * row_chunks;
        for (int c0 = tid; c0 < total; c0 += 4 * 256) {
            u32x4_t v[4];
            int pr[4], rc[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + 256 * u;
                pr[u] = c / row_chunks;
                rc[u] = c - pr[u] * row_chunks;
                const int hi = hi0 + pr[u];
                ok[u] = c < total && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H);   // else stays zero
                if (ok[u]) v[u] = *reinterpret_cast<const u32x4_t*>(xb + (static_cast<int64_t>(hi) * row_vals + 8 * rc[u]) * 2);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!ok[u]) continue;
                const int idx = 8 * rc[u];
                int wi = idx / p.Cin, ci = idx - wi * p.Cin;
                uint8_t* const rowp = sx + (pr[u] * p.pw + p.PW) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t word = v[u][e >> 1];
                    const uint16_t val = static_cast<uint16_t>((e & 1) ? (word >> 16) : (word & 0xFFFFu));
                    *reinterpret_cast<uint16_t*>(rowp + (wi * 4 + ci) * 2) = val;
                    if (++ci == p.Cin) {
                        ci = 0;
                        ++wi;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- 32-pixel fragments, two at a time per wave (fragments f and f + 4), so that four
    //      accumulator chains interleave on the matrix pipe ----
    const int npx = rows * p.Wo;
    const int nfrag = (npx + 31) / 32;
    const int ksteps = p.kwp / 4;                           // 1 .. 4 (the host bounds KH * kwp)
    const int nj = nco / 32;
    uint8_t* const yb = reinterpret_cast<uint8_t*>(p.y);
    const uint8_t* const bbase = sw + (lane & 31) * wstride + 2 * half * 8;
    const int bstep_j = 32 * wstride;
    uint8_t* const stg = smem + kSmallLds + wave * kSmallStage;
    const int cpr = nco / 8;                                // 16-byte chunks of a staged row
    for (int f0 = wave; f0 < nfrag; f0 += 8) {
        int hl[2], wo[2];
        bool pv[2];
        const uint8_t* abase[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pl = (f0 + 4 * u) * 32 + (lane & 31);
            pv[u] = pl < npx;
            const int plc = pv[u] ? pl : 0;
            hl[u] = plc / p.Wo;
            wo[u] = plc - hl[u] * p.Wo;
            abase[u] = sx + ((hl[u] * p.SH) * p.pw + wo[u] * p.SW + 2 * half) * 8;
        }
        f32x16_t acc[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[u][j][e] = 0.0f;
        for (int r = 0; r < p.KH; ++r) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks >= ksteps) break;
                bf16x8_t av[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint8_t* const a = abase[u] + (r * p.pw + 4 * ks) * 8;
                    const uint2 a0 = *reinterpret_cast<const uint2*>(a);
                    const uint2 a1 = *reinterpret_cast<const uint2*>(a + 8);
                    av[u] = __builtin_bit_cast(bf16x8_t, u32x4_t{a0.x, a0.y, a1.x, a1.y});
                }
                const uint8_t* const b = bbase + (r * p.kwp + 4 * ks) * 8;
                const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(b);
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, av[0], acc[0][0], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, av[1], acc[1][0], 0, 0, 0);
                if (nj > 1) {
                    const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(b + bstep_j);
                    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, av[0], acc[0][1], 0, 0, 0);
                    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, av[1], acc[1][1], 0, 0, 0);
                }
            }
        }
        // lane: pixel of fragment f0 + 4u; register group g of channel fragment j holds
        // channels 32 j + 8 g + 4 half .. +3.  The finished fragment goes through this wave's
        // staging area, 32 rows of 128 bytes with chunk c of row m at c ^ ((m >> 1) & 7), and
        // out as whole rows of 16-byte stores.
        const int m = lane & 31, swz = (m >> 1) & 7;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int f = f0 + 4 * u;
            if (f >= nfrag) break;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (j >= nj) break;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int co = co0 + 32 * j + 8 * g + 4 * half;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[u][j][4 * g + e];
                    if (p.bias) {
                        const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(p.bias + co);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] += bv[e];
                    }
                    if constexpr (RES) {
                        if (pv[u]) {
                            const int64_t pix = (static_cast<int64_t>(img) * p.Ho + ho0 + hl[u]) * p.Wo + wo[u];
                            const uint2 rv = *reinterpret_cast<const uint2*>(p.res + pix * p.Cout + co);
                            v[0] += __uint_as_float(rv.x << 16);
                            v[1] += __uint_as_float(rv.x & 0xFFFF0000u);
                            v[2] += __uint_as_float(rv.y << 16);
                            v[3] += __uint_as_float(rv.y & 0xFFFF0000u);
                        }
                    }
                    if constexpr (ACT == kActGelu || ACT == kActGeluErf) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = activate<ACT>(v[e]);
                    }
                    uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
                    if constexpr (ACT == kActRelu) {
                        lo = relu_bf16x2(lo);
                        hi = relu_bf16x2(hi);
                    }
                    *reinterpret_cast<uint2*>(stg + m * 128 + (((4 * j + g) ^ swz) << 4) + 8 * half) = make_uint2(lo, hi);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's staging writes are done
            __builtin_amdgcn_wave_barrier();
            // rows of the fragment: pixel f 32 + r of the tile, cpr chunks each
            for (int q = lane; q < 32 * cpr; q += 64) {
                const int r = q / cpr, c = q - r * cpr;
                const int pl = f * 32 + r;
                if (pl >= npx) continue;
                const int hr = pl / p.Wo, wr = pl - hr * p.Wo;
                const int64_t pix = (static_cast<int64_t>(img) * p.Ho + ho0 + hr) * p.Wo + wr;
                const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stg + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
                *reinterpret_cast<u32x4_t*>(yb + (pix * p.Cout + co0 + 8 * c) * 2) = val;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // the staging reads are done before the next writes
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int ACT>
hipError_t launch_act(const SmallCArgs& a, dim3 grid, hipStream_t s) {
    if (a.res)
        hipLaunchKernelGGL((conv_smallc_kernel<ACT, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((conv_smallc_kernel<ACT, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool conv_smallc_plan(int N, int H, int W, int Cin, int Cout, int KH, int KW, int SH, int SW, int PH, int PW,
                      int Ho, int Wo, SmallCArgs* a) {
    if (Cin < 1 || Cin > 4 || Cout < 32 || Cout % 32 != 0 || N < 1 || H < 1 || W < 1 || Ho < 1 || Wo < 1)
        return false;
    if ((W * Cin) % 8 != 0) return false;                 // whole 16-byte chunks per input row
    const int kwp = (KW + 3) / 4 * 4;
    if (kwp > 16) return false;                            // at most four MFMA steps per kernel row
    const int wbytes = 64 * smallc_wstride(KH, kwp);
    if (wbytes > kSmallLds / 2) return false;
    // patch columns: every input column (filled) and every column a fragment reads, padded
    // taps included
    int pw = W + PW > (Wo - 1) * SW + kwp ? W + PW : (Wo - 1) * SW + kwp;
    pw = (pw + 1) / 2 * 2;
    const int rows_fit = (kSmallLds - wbytes) / (pw * 8);
    if (rows_fit < KH) return false;
    int th = (rows_fit - KH) / SH + 1;                     // th rows read (th - 1) SH + KH input rows
    th = th > 16 ? 16 : th;
    th = th > Ho ? Ho : th;
    a->N = N; a->H = H; a->W = W; a->Cin = Cin; a->Cout = Cout;
    a->KH = KH; a->KW = KW; a->SH = SH; a->SW = SW; a->PH = PH; a->PW = PW;
    a->Ho = Ho; a->Wo = Wo;
    a->kwp = kwp;
    a->pw = pw;
    a->th = th;
    a->row_tiles = (Ho + th - 1) / th;
    a->co_blocks = (Cout + 63) / 64;
    return true;
}

hipError_t launch_conv_smallc(const SmallCArgs& a, int act, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(a.N) * a.row_tiles * a.co_blocks;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (act) {
        case kActNone: return launch_act<kActNone>(a, grid, s);
        case kActRelu: return launch_act<kActRelu>(a, grid, s);
        case kActGelu: return launch_act<kActGelu>(a, grid, s);
        case kActGeluErf: return launch_act<kActGeluErf>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlf
