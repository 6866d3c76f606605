// bf16 convolution for images with few channels (c_in <= 4, such as the 3-channel input of
// a ResNet stem: 7x7, stride 2, pad 3) with the register epilogue of the fused operator
// (bias -> residual -> activation -> one rounding, each output element stored once; the
// conv epilogue of "OpenPPL算子融合深度解析" §4.3 with the folded BN of §3.1).
//
// A 16-byte-chunk implicit GEMM wastes most of its loads here: a chunk of 8 k-values spans
// several taps and is not aligned.  Instead one workgroup per CU keeps in LDS
//   - its 64 output channels' weights as [co][r][t][4 channels], t = s + toff the kernel
//     column shifted so that the image's column 0 falls on an even patch column (toff is 1
//     for an odd left padding), zero outside the kernel and in channels past c_in,
//   - the input patch under its output rows as [row][column][4 channels] (8 bytes a pixel),
//     the image's column 0 at the even column pwl, zero outside the image,
// so that one lane's 8 k-values of a 32x32x16 MFMA (two neighbouring taps t, t+1 of one
// kernel row, four channels each) are 16 contiguous bytes in both, 16-byte aligned in the
// patch when the column stride is even.  Both are written once, without a zero fill: a
// thread loads whole input pixel pairs (c_in dwords, dword-aligned because pairs start at
// even image columns) and writes them out widened to four channels, each weight tap comes
// from one 8-byte load shifted into place, and positions outside the image or the kernel
// come from loads past the buffer, which read 0.  Before the first K loop only the weights
// and the patch rows of the first round are filled; the store waves, which have nothing to
// store in the first round, fill the other rows meanwhile.
//
// What bounds this layer is its output: 64 output channels from 3 input channels make
// 51 MB written against 10 MB read for a batch of 32 224x224 images.  The workgroup
// therefore splits its 16 waves by role.  Eight compute waves (two per SIMD) run the K
// loop for two 32-pixel fragments each per round and leave the finished fragments in LDS;
// eight store waves copy a round's fragments out to memory while the compute waves run the
// next round.  When every wave stores its own fragments, all of them stall on the full
// store queue after each fragment, and the stores come in bursts separated by stretches of
// K loop with no store in flight.
#include "device_common.h"
#include "kernels.h"
#include "mma_common.h"

namespace dlf {
namespace {

constexpr int kScLds = 160 * 1024;                  // the CU's whole LDS: one workgroup per CU
constexpr int kScThreads = 1024;                    // 16 waves
constexpr int kScCompute = 8;                       // compute waves, two per SIMD; the rest store
constexpr int kScRound = 2 * kScCompute;            // 32-pixel fragments a round
constexpr int kScFrag = 32 * 128;                   // one staged fragment: 32 rows of 64 channels
constexpr int kScStage = kScRound * kScFrag;        // 64 KB
constexpr int kScBias = 64 * 4;                     // the workgroup's 64 biases, fp32

// bytes between two output channels' weights: KH kwp 8, plus 16 where that is an even number
// of 16-byte chunks, so that the 32 lanes' fragment reads (one channel each) fall in distinct
// LDS banks
__host__ __device__ inline int smallc_wstride(int kh, int kwp) {
    const int b = kh * kwp * 8;
    return (b / 16) % 2 == 0 ? b + 16 : b;
}

// s_waitcnt lgkmcnt(0), then s_barrier: this wave's LDS reads and writes are done before the
// other waves pass.  Outstanding global stores are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier();
}

// a / b for 0 <= a < 2^22 and b >= 1 given inv = 1 / b: (a + 1/2) / b lies at least 1 / (2b)
// from an integer, and the two float roundings move it by at most (a + 1/2) / b * 2^-23
__device__ __forceinline__ int small_div(int a, float inv) {
    return static_cast<int>((static_cast<float>(a) + 0.5f) * inv);
}

// One lane's 8 k-values of a pixel fragment: 16 bytes of the patch, 16-byte aligned when the
// column stride is even (A16), else 8-byte aligned.
template <bool A16>
__device__ __forceinline__ bf16x8_t read_a(const uint8_t* a) {
    if constexpr (A16) {
        return *reinterpret_cast<const bf16x8_t*>(a);
    } else {
        const uint2 a0 = *reinterpret_cast<const uint2*>(a);
        const uint2 a1 = *reinterpret_cast<const uint2*>(a + 8);
        return __builtin_bit_cast(bf16x8_t, u32x4_t{a0.x, a0.y, a1.x, a1.y});
    }
}

// CIN consecutive dwords of buffer r at byte offset off (zeros past the buffer)
template <int CIN>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* d) {
    if constexpr (CIN == 1) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (CIN == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        d[0] = v[0]; d[1] = v[1];
    } else if constexpr (CIN == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2];
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    }
}

// two input pixels of CIN bf16 channels each (CIN dwords) as two 8-byte pixels of 4 channels
template <int CIN>
__device__ __forceinline__ u32x4_t widen_pair(const uint32_t* d) {
    if constexpr (CIN == 1) return u32x4_t{d[0] & 0xFFFFu, 0u, d[0] >> 16, 0u};
    else if constexpr (CIN == 2) return u32x4_t{d[0], 0u, d[1], 0u};
    else if constexpr (CIN == 3) return u32x4_t{d[0], d[1] & 0xFFFFu, (d[1] >> 16) | (d[2] << 16), d[2] >> 16};
    else return u32x4_t{d[0], d[1], d[2], d[3]};
}

// Weights of channels co0 .. co0+nco-1 re-laid as [co][r][t][4 channels] and the first
// rows of the input patch, every position written once.  Weight chunk (co, r, tp) holds taps
// t = 2 tp and 2 tp + 1 of kernel row r: each tap's CIN channels come from one 8-byte load
// that lies wholly inside the block (from the dword below them, or from the block's last
// 8 bytes), shifted down to them; a tap outside the kernel reads past the buffer: zero.  Each
// pass issues the loads of two weight chunks and four pixel pairs a thread before any LDS
// write.
template <int CIN>
__device__ void smallc_fill(const SmallCArgs& p, uint8_t* sw, uint8_t* sx, int wstride, int img, int co0, int nco,
                            int hi0, int prows0, int tid) {
    const int kp2 = p.kwp / 2, per_co = p.KH * kp2, wchunks = nco * per_co;
    const float inv_co = 1.0f / static_cast<float>(per_co), inv_kp2 = 1.0f / static_cast<float>(kp2);
    const int kvals = p.KH * p.KW * CIN;
    const uint32_t wbytes = static_cast<uint32_t>(nco * kvals * 2);   // a multiple of 64
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(p.w + static_cast<int64_t>(co0) * kvals, wbytes);
    const int pairs = p.pw / 2;
    const int64_t img_bytes = static_cast<int64_t>(p.H) * p.W * CIN * 2;
    const __amdgpu_buffer_rsrc_t xr =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.x) + img * img_bytes, static_cast<uint32_t>(img_bytes));
    const float inv_pairs = 1.0f / static_cast<float>(pairs);
    int pr = small_div(tid, inv_pairs), cp = tid - pr * pairs;
    const int dpr = small_div(kScThreads, inv_pairs), dcp = kScThreads - dpr * pairs;
    for (int c0 = tid; c0 < wchunks || pr < prows0; c0 += 2 * kScThreads) {
        uint64_t wv[2][2];
        uint32_t wsh[2][2];
        int wdst[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = c0 + k * kScThreads;
            const int co = small_div(c, inv_co), rem = c - co * per_co;
            const int r = small_div(rem, inv_kp2), tp = rem - r * kp2;
            wdst[k] = c < wchunks ? co * wstride + (r * p.kwp + 2 * tp) * 8 : -1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int s = 2 * tp + h - p.toff;
                const bool ok = c < wchunks && s >= 0 && s < p.KW;
                const uint32_t off = static_cast<uint32_t>(((co * p.KH + r) * p.KW + s) * CIN * 2);
                const uint32_t base = min(off & ~3u, wbytes - 8u);
                wsh[k][h] = (off - base) * 8u;
                const auto d = __builtin_amdgcn_raw_buffer_load_b64(wr, ok ? base : kOutOfRange, 0, 0);
                wv[k][h] = static_cast<uint64_t>(d[0]) | (static_cast<uint64_t>(d[1]) << 32);
            }
        }
        uint32_t d[4][CIN];
        int dst[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool live = pr < prows0;
            const int hi = hi0 + pr, w = 2 * cp - p.pwl;
            const bool in = live && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                            static_cast<unsigned>(w) < static_cast<unsigned>(p.W);
            load_dwords<CIN>(xr, in ? static_cast<uint32_t>((hi * p.W + w) * CIN * 2) : kOutOfRange, d[u]);
            dst[u] = live ? (pr * p.pw + 2 * cp) * 8 : -1;
            cp += dcp;
            pr += dpr;
            if (cp >= pairs) {
                cp -= pairs;
                ++pr;
            }
        }
        constexpr uint64_t kMask = CIN == 4 ? ~uint64_t(0) : (uint64_t(1) << (16 * CIN)) - 1;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (wdst[k] < 0) continue;
            const uint64_t t0 = (wv[k][0] >> wsh[k][0]) & kMask, t1 = (wv[k][1] >> wsh[k][1]) & kMask;
            *reinterpret_cast<u32x4_t*>(sw + wdst[k]) = u32x4_t{static_cast<uint32_t>(t0), static_cast<uint32_t>(t0 >> 32),
                                                                static_cast<uint32_t>(t1), static_cast<uint32_t>(t1 >> 32)};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (dst[u] >= 0) *reinterpret_cast<u32x4_t*>(sx + dst[u]) = widen_pair<CIN>(d[u]);
    }
}

// Patch rows pr_begin .. pr_end-1 (image rows hi0 + pr) into their LDS layout, by threads
// t = 0 .. nthr-1.  Pair (pr, cp) is patch columns 2 cp, 2 cp + 1 = image columns
// 2 cp - pwl (even) and the next one.  Four pairs a thread per pass, their loads in flight
// together; the pair index steps by nthr without a division.
template <int CIN>
__device__ void smallc_fill_patch(const SmallCArgs& p, uint8_t* sx, int img, int hi0, int pr_begin, int pr_end,
                                  int t, int nthr) {
    const int pairs = p.pw / 2;
    const int64_t img_bytes = static_cast<int64_t>(p.H) * p.W * CIN * 2;
    const __amdgpu_buffer_rsrc_t xr =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.x) + img * img_bytes, static_cast<uint32_t>(img_bytes));
    const float inv_pairs = 1.0f / static_cast<float>(pairs);
    int pr = small_div(t, inv_pairs), cp = t - pr * pairs;
    pr += pr_begin;
    const int dpr = small_div(nthr, inv_pairs), dcp = nthr - dpr * pairs;
    while (pr < pr_end) {
        uint32_t d[4][CIN];
        int dst[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool live = pr < pr_end;
            const int hi = hi0 + pr, w = 2 * cp - p.pwl;
            const bool in = live && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                            static_cast<unsigned>(w) < static_cast<unsigned>(p.W);
            load_dwords<CIN>(xr, in ? static_cast<uint32_t>((hi * p.W + w) * CIN * 2) : kOutOfRange, d[u]);
            dst[u] = live ? (pr * p.pw + 2 * cp) * 8 : -1;
            cp += dcp;
            pr += dpr;
            if (cp >= pairs) {
                cp -= pairs;
                ++pr;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (dst[u] >= 0) *reinterpret_cast<u32x4_t*>(sx + dst[u]) = widen_pair<CIN>(d[u]);
    }
}

__device__ __forceinline__ void smallc_fill_patch_any(const SmallCArgs& p, uint8_t* sx, int img, int hi0,
                                                      int pr_begin, int pr_end, int t, int nthr) {
    switch (p.Cin) {
        case 1: smallc_fill_patch<1>(p, sx, img, hi0, pr_begin, pr_end, t, nthr); break;
        case 2: smallc_fill_patch<2>(p, sx, img, hi0, pr_begin, pr_end, t, nthr); break;
        case 3: smallc_fill_patch<3>(p, sx, img, hi0, pr_begin, pr_end, t, nthr); break;
        default: smallc_fill_patch<4>(p, sx, img, hi0, pr_begin, pr_end, t, nthr); break;
    }
}

template <int ACT, bool RES, bool A16>
__global__ __launch_bounds__(kScThreads, 1) void conv_smallc_kernel(const SmallCArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kScLds];
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
    uint8_t* const stage = smem;
    float* const sbias = reinterpret_cast<float*>(smem + kScStage);
    uint8_t* const sw = smem + kScStage + kScBias;
    uint8_t* const sx = sw + 64 * wstride;

    // ---- fill: biases, weights, the first round's patch rows.  The bias load goes out first
    //      and lands in LDS after the fill, so that its latency hides behind the fill's. ----
    f32x4_t bias4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tid < 16 && p.bias && 4 * tid < nco) bias4 = *reinterpret_cast<const f32x4_t*>(p.bias + co0 + 4 * tid);
    const int npx = rows * p.Wo;                            // the tile's pixels: whole output rows,
    const int nfrag = (npx + 31) / 32;                      // contiguous in y
    const int nrounds = (nfrag + kScRound - 1) / kScRound;
    // patch rows: the first round's fragments read rows 0 .. prows0-1, filled now; the store
    // waves fill the rest during the first round, in which they have nothing to store
    const int hi0 = ho0 * p.SH - p.PH;
    const int prows = (rows - 1) * p.SH + p.KH;
    const int prows0 = min(prows, ((min(npx, kScRound * 32) - 1) / p.Wo) * p.SH + p.KH);
    switch (p.Cin) {
        case 1: smallc_fill<1>(p, sw, sx, wstride, img, co0, nco, hi0, prows0, tid); break;
        case 2: smallc_fill<2>(p, sw, sx, wstride, img, co0, nco, hi0, prows0, tid); break;
        case 3: smallc_fill<3>(p, sw, sx, wstride, img, co0, nco, hi0, prows0, tid); break;
        default: smallc_fill<4>(p, sw, sx, wstride, img, co0, nco, hi0, prows0, tid); break;
    }
    if (tid < 16) *reinterpret_cast<f32x4_t*>(sbias + 4 * tid) = bias4;
    lds_barrier();   // weights, biases and the first round's patch rows are in place

    const int64_t pix0 = (static_cast<int64_t>(img) * p.Ho + ho0) * p.Wo;
    const int cpr = nco / 8;                                // 16-byte chunks of a pixel's channels

    if (wave < kScCompute) {
        // ---- compute waves: fragments f0 and f0 + 8 of each round, four accumulator chains
        //      (2 fragments x 2 channel halves) interleaved on the matrix pipe ----
        const int ksteps = p.kwp / 4;                       // 1 .. 4
        const int nj = nco / 32;                            // channel halves staged
        const uint8_t* const bbase = sw + (lane & 31) * wstride + 2 * half * 8;
        const int bstep_j = 32 * wstride;
        const int m = lane & 31, swz = (m >> 1) & 7;
        const float inv_wo = 1.0f / static_cast<float>(p.Wo);
        for (int rd = 0; rd < nrounds; ++rd) {
            const int f0 = rd * kScRound + wave;
            const bool any = f0 < nfrag;
            f32x16_t acc[2][2];
            int pl[2];
            bool pv[2];
            if (any) {
                const uint8_t* abase[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int q = (f0 + 8 * u) * 32 + m;
                    pv[u] = q < npx;
                    pl[u] = pv[u] ? q : 0;
                    const int hl = small_div(pl[u], inv_wo), wo = pl[u] - hl * p.Wo;
                    abase[u] = sx + ((hl * p.SH) * p.pw + wo * p.SW + 2 * half) * 8;
                }
                // the accumulators start at the bias: the epilogue then reads nothing from LDS
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(sbias + 32 * j + 8 * g + 4 * half);
#pragma unroll
                        for (int u = 0; u < 2; ++u)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[u][j][4 * g + e] = bv[e];
                    }
                // k-step i reads kernel row i / ksteps, taps 4 (i % ksteps) .. +3: 32 bytes on
                // within a row, to the next row's start after its last step.  The next step's
                // operands are read before this step's four MFMAs.  Both channel halves are
                // computed; with 32 channels the second is never staged.
                const int nk = p.KH * ksteps;
                const int a_row = (p.pw - 4 * (ksteps - 1)) * 8, b_row = (p.kwp - 4 * (ksteps - 1)) * 8;
                const uint8_t* pa0 = abase[0];
                const uint8_t* pa1 = abase[1];
                const uint8_t* pb = bbase;
                bf16x8_t a0 = read_a<A16>(pa0), a1 = read_a<A16>(pa1);
                bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(pb), b1 = *reinterpret_cast<const bf16x8_t*>(pb + bstep_j);
                int ks = 0;
                for (int i = 0; i < nk; ++i) {
                    bf16x8_t na0 = a0, na1 = a1, nb0 = b0, nb1 = b1;
                    if (i + 1 < nk) {
                        const bool row_end = ++ks == ksteps;
                        if (row_end) ks = 0;
                        const int da = row_end ? a_row : 32, db = row_end ? b_row : 32;
                        pa0 += da;
                        pa1 += da;
                        pb += db;
                        na0 = read_a<A16>(pa0);
                        na1 = read_a<A16>(pa1);
                        nb0 = *reinterpret_cast<const bf16x8_t*>(pb);
                        nb1 = *reinterpret_cast<const bf16x8_t*>(pb + bstep_j);
                    }
                    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, a0, acc[0][0], 0, 0, 0);
                    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, a1, acc[1][0], 0, 0, 0);
                    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, a0, acc[0][1], 0, 0, 0);
                    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, a1, acc[1][1], 0, 0, 0);
                    a0 = na0;
                    a1 = na1;
                    b0 = nb0;
                    b1 = nb1;
                }
            }
            lds_barrier();   // B1: the store waves hold the previous round's fragments
            if (any) {
                // lane: pixel m of its fragment; register group g of channel half j holds
                // channels 32 j + 8 g + 4 half .. +3.  Staged as 32 rows of 128 bytes with
                // chunk c of row m at c ^ ((m >> 1) & 7).
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (f0 + 8 * u >= nfrag) break;
                    uint8_t* const stg = stage + (2 * wave + u) * kScFrag;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (j >= nj) break;
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int col = 32 * j + 8 * g + 4 * half;
                            float v[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = acc[u][j][4 * g + e];
                            if constexpr (RES) {
                                if (pv[u]) {
                                    const uint2 rv = *reinterpret_cast<const uint2*>(
                                        p.res + (pix0 + pl[u]) * p.Cout + co0 + col);
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
                            *reinterpret_cast<uint2*>(stg + m * 128 + (((4 * j + g) ^ swz) << 4) + 8 * half) =
                                make_uint2(lo, hi);
                        }
                    }
                }
            }
            lds_barrier();   // B2: this round's fragments are staged
        }
    } else {
        // ---- store waves: wave 8 + s copies the fragments of compute wave s (staging slots
        //      2 s and 2 s + 1), 16 bytes a lane per row chunk, into registers after B2 and
        //      out to y during the next round.  Stores write through to device scope: every
        //      store instruction covers whole 128-byte lines, and no dirty lines are left for
        //      the end of the kernel. ----
        const int s = wave - kScCompute;
        const int shift = cpr == 8 ? 3 : 2;
        const __amdgpu_buffer_rsrc_t yr = buffer_rsrc(reinterpret_cast<uint8_t*>(p.y) + (pix0 * p.Cout + co0) * 2,
                                                      static_cast<uint32_t>(npx * p.Cout * 2));
        u32x4_t held[2][4];
        auto store_round = [&](int rd) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int f = rd * kScRound + s + 8 * u;
                if (f >= nfrag) break;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (2 * i >= cpr) break;
                    const int q = lane + 64 * i, row = q >> shift, c = q & (cpr - 1);
                    const int px = f * 32 + row;
                    if (px < npx)
                        __builtin_amdgcn_raw_buffer_store_b128(held[u][i], yr,
                                                               static_cast<uint32_t>((px * p.Cout + 8 * c) * 2), 0,
                                                               kStoreDevice);
                }
            }
        };
        smallc_fill_patch_any(p, sx, img, hi0, prows0, prows, tid - kScCompute * 64, kScThreads - kScCompute * 64);
        for (int rd = 0; rd < nrounds; ++rd) {
            if (rd > 0) store_round(rd - 1);
            lds_barrier();   // B1
            lds_barrier();   // B2
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int f = rd * kScRound + s + 8 * u;
                if (f >= nfrag) break;
                const uint8_t* const stg = stage + (2 * s + u) * kScFrag;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (2 * i >= cpr) break;
                    const int q = lane + 64 * i, row = q >> shift, c = q & (cpr - 1);
                    held[u][i] = *reinterpret_cast<const u32x4_t*>(stg + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
                }
            }
        }
        store_round(nrounds - 1);
    }
}

template <int ACT, bool RES>
hipError_t launch_res(const SmallCArgs& a, dim3 grid, hipStream_t s) {
    if (a.SW % 2 == 0)
        hipLaunchKernelGGL((conv_smallc_kernel<ACT, RES, true>), grid, dim3(kScThreads), 0, s, a);
    else
        hipLaunchKernelGGL((conv_smallc_kernel<ACT, RES, false>), grid, dim3(kScThreads), 0, s, a);
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_act(const SmallCArgs& a, dim3 grid, hipStream_t s) {
    return a.res ? launch_res<ACT, true>(a, grid, s) : launch_res<ACT, false>(a, grid, s);
}

}  // namespace

bool conv_smallc_plan(int N, int H, int W, int Cin, int Cout, int KH, int KW, int SH, int SW, int PH, int PW,
                      int Ho, int Wo, SmallCArgs* a) {
    if (Cin < 1 || Cin > 4 || Cout < 32 || Cout % 32 != 0 || N < 1 || H < 1 || W < 1 || Ho < 1 || Wo < 1)
        return false;
    if ((W * Cin) % 8 != 0) return false;                 // W even: a pixel pair never straddles a row
    if (static_cast<int64_t>(H) * W * Cin * 2 >= (int64_t(1) << 31)) return false;   // 32-bit offsets in an image
    const int pwl = PW + (PW & 1), toff = pwl - PW;
    const int kwp = (KW + toff + 3) / 4 * 4;
    if (kwp > 16) return false;                            // at most four MFMA steps per kernel row
    const int wbytes = 64 * smallc_wstride(KH, kwp);
    // patch columns: every column a fragment reads, wo SW + t for t < kwp
    const int pw = ((Wo - 1) * SW + kwp + 1) / 2 * 2;
    const int budget = kScLds - kScStage - kScBias - wbytes;
    if (budget <= 0 || pw > 4096) return false;
    const int rows_fit = budget / (pw * 8);
    if (rows_fit < KH) return false;
    const int th_max = (rows_fit - KH) / SH + 1;           // th rows read (th - 1) SH + KH input rows
    const int co_blocks = (Cout + 63) / 64;
    // as few row tiles as the LDS allows, but at least one workgroup per CU where the rows
    // allow it, and the rows shared out evenly
    int row_tiles = (Ho + th_max - 1) / th_max;
    const int64_t per_img = static_cast<int64_t>(N) * co_blocks;
    const int64_t want = (256 + per_img - 1) / per_img;
    if (row_tiles < want) row_tiles = static_cast<int>(want < Ho ? want : Ho);
    const int th = (Ho + row_tiles - 1) / row_tiles;
    if (static_cast<int64_t>(th) * Wo * Cout * 2 >= (int64_t(1) << 31)) return false;   // 32-bit store offsets
    if (static_cast<int64_t>(N) * ((Ho + th - 1) / th) * co_blocks > 0x7FFFFFFF) return false;
    a->N = N; a->H = H; a->W = W; a->Cin = Cin; a->Cout = Cout;
    a->KH = KH; a->KW = KW; a->SH = SH; a->SW = SW; a->PH = PH; a->PW = PW;
    a->Ho = Ho; a->Wo = Wo;
    a->kwp = kwp;
    a->pw = pw;
    a->pwl = pwl;
    a->toff = toff;
    a->th = th;
    a->row_tiles = (Ho + th - 1) / th;
    a->co_blocks = co_blocks;
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
