// Transformer feed-forward block in one kernel, FC1 -> activation -> FC2, with the activated
// intermediate kept on chip (the FFN fusion of "OpenPPL算子融合深度解析" §3.2; the second
// layer's bias and the block's residual add ride in its epilogue, §3.3):
//     y = act(x W1^T + b1) W2^T + b2 [+ residual]
//
// A workgroup owns 32 or 64 tokens and every one of the d_model output columns, so no partial
// sum leaves the chip.  It walks d_ff in chunks of 256:
//   FC1: wave w computes h[32 tokens][32 features] = act(x W1[f]^T + b1) for the chunk's
//        features 32w .. 32w+31 over all of d_model (x resident in LDS), rounds it to bf16
//        and puts it in LDS (double-buffered, one barrier per chunk);
//   FC2: wave w accumulates its d_model/8 output columns over the chunk's 256 features.
// The tokens x d_model fp32 accumulator stays in registers for the whole walk.  The weights are
// streamed from L2/HBM in MFMA fragment order (packed once at load time, see dlf_ffn_pack):
// each wave's fragment of a 32x32x16 MFMA is one contiguous kilobyte, fetched many
// (16 or 32) fragments ahead into a register ring.  Every weight byte is read once per workgroup, so the
// weight traffic through L2 falls with the tokens a workgroup owns.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "mma_common.h"

namespace dlf {
namespace {

constexpr int kChunk = 256;        // d_ff features per chunk (8 waves x 32)
constexpr int kHPitch = kChunk * 2 + 16;       // bytes per token row of h in LDS (padded)

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), unrolled at compile time
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for_from(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    static_for_from<0, N>(f);
}

// DB: 32-column output blocks per wave (d_model = 256 DB); FT: 32-token fragments per
// workgroup.  With FT = 2 the weights are read once per 64 tokens (half the L2 traffic of
// FT = 1) and the h buffer is single (LDS), which costs a second barrier per chunk.
// SPL: d_ff split into S = p.parts parts: workgroup S b + part takes token block b and the
// chunks [part nchunks / S, (part + 1) nchunks / S), and writes its fp32 partial sum of y (no
// bias, no residual) to p.ws[part]; ffn_reduce_kernel finishes y.  Each workgroup then
// streams 1/S of the weights for its tokens.
template <int ACT, int DB, int FT, bool SPL>
__global__ __launch_bounds__(512, 1) void ffn_kernel(const FfnArgs p) {
    // weight fragments in flight per wave: the stream is latency-bound, so as many as the
    // registers allow (4 a fragment beside the FT x DB accumulators)
    constexpr int kRing = FT == 1 && (DB == 1 || DB == 3) ? 32 : 16;
    constexpr int D = 256 * DB;
    constexpr int TOK = 32 * FT;
    constexpr int XP = D * 2 + 16;              // bytes per token row of x in LDS (padded)
    constexpr int NB = FT == 1 ? 2 : 1;         // h buffers
    __shared__ __attribute__((aligned(16))) uint8_t xs[TOK * XP];
    __shared__ __attribute__((aligned(16))) uint8_t hs[NB][TOK * kHPitch];
    constexpr int KS1 = D / 16;                 // FC1 k-steps (over d_model)
    constexpr int KS2 = kChunk / 16;            // FC2 k-steps per chunk (over d_ff)
    constexpr int QN = KS1 + KS2 * DB;          // weight fragments per wave per chunk
    static_assert(QN % kRing == 0, "the ring index repeats from chunk to chunk");
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, tok = lane & 31;
    const int S = SPL ? p.parts : 1;
    const int part = static_cast<int>(blockIdx.x % static_cast<unsigned>(S));
    const int64_t m0 = static_cast<int64_t>(blockIdx.x / static_cast<unsigned>(S)) * TOK;
    const int F = p.F;
    const int nchunks = F / kChunk;
    const int cbeg = part * nchunks / S, cend = (part + 1) * nchunks / S;   // this part's chunks (S <= nchunks)

    // ---- x rows m0 .. m0+TOK-1 into LDS (zero past M) ----
    for (int i = tid; i < TOK * (D / 8); i += 512) {
        const int t = i / (D / 8), c = i - t * (D / 8);
        u32x4_t v{0u, 0u, 0u, 0u};
        if (m0 + t < p.M) v = *reinterpret_cast<const u32x4_t*>(p.x + (m0 + t) * D + 8 * c);
        *reinterpret_cast<u32x4_t*>(xs + t * XP + 16 * c) = v;
    }

    // weight fragment q of chunk c for this wave: q < KS1 is FC1 step q of feature block
    // 8c + wave; then FC2 step (q - KS1) / DB of output block wave*DB + (q - KS1) % DB
    const int ks_f = F / 16;
    auto frag = [&](int c, int q) -> const u32x4_t* {
        int64_t idx;
        if (q < KS1) {
            idx = (static_cast<int64_t>(8 * c + wave) * KS1 + q) * 64 + lane;
            return reinterpret_cast<const u32x4_t*>(p.w1p) + idx;
        }
        const int s = (q - KS1) / DB, b = (q - KS1) - s * DB;
        idx = (static_cast<int64_t>(wave * DB + b) * ks_f + c * KS2 + s) * 64 + lane;
        return reinterpret_cast<const u32x4_t*>(p.w2p) + idx;
    };
    u32x4_t ring[kRing];
#pragma unroll
    for (int q = 0; q < kRing; ++q) ring[q] = *frag(cbeg, q);

    f32x16_t acc2[DB][FT];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc2[b][f][e] = 0.0f;
    __syncthreads();

    for (int c = cbeg; c < cend; ++c) {
        uint8_t* const hbuf = hs[NB == 2 ? (c & 1) : 0];
        // FC1 accumulators: FT token fragments, each split over even and odd k-steps when there
        // is only one, so that two independent chains keep the matrix pipe busy
        constexpr int SPLIT = FT == 1 ? 2 : 1;
        f32x16_t acc1[FT][SPLIT];
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
            for (int h = 0; h < SPLIT; ++h)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc1[f][h][e] = 0.0f;
        // weight fragment q is consumed from ring slot q % kRing, which is then refilled with
        // fragment q + kRing (the next chunk's first ones near the end)
        auto take = [&](auto q_c) -> bf16x8_t {
            constexpr int q = decltype(q_c)::value;
            const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, ring[q % kRing]);
            if constexpr (q + kRing < QN) {
                ring[q % kRing] = *frag(c, q + kRing);
            } else {
                if (c + 1 < cend) ring[q % kRing] = *frag(c + 1, q + kRing - QN);
            }
            return wv;
        };
        static_for<KS1>([&](auto q_c) {
            constexpr int q = decltype(q_c)::value;
            const bf16x8_t wv = take(q_c);
#pragma unroll
            for (int f = 0; f < FT; ++f) {
                const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(xs + (32 * f + tok) * XP + 16 * half + 32 * q);
                acc1[f][q % SPLIT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, xv, acc1[f][q % SPLIT], 0, 0, 0);
            }
        });
        if constexpr (NB == 1) {
            // one h buffer: every wave must be done reading the previous chunk's h
            if (c > cbeg) {
                wait_vm_lgkm<63, 0>();
                barrier();
            }
        }
        // FC1 epilogue: lane holds token 32 f + tok, features 32 wave + 8 g + 4 half .. +3
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int fl = 32 * wave + 8 * g + 4 * half;
            f32x4_t bv{0.0f, 0.0f, 0.0f, 0.0f};
            if (p.b1) bv = *reinterpret_cast<const f32x4_t*>(p.b1 + c * kChunk + fl);
#pragma unroll
            for (int f = 0; f < FT; ++f) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a = acc1[f][0][4 * g + e];
                    if constexpr (SPLIT == 2) a += acc1[f][SPLIT - 1][4 * g + e];
                    v[e] = activate<ACT>(a + bv[e]);
                }
                *reinterpret_cast<uint2*>(hbuf + (32 * f + tok) * kHPitch + 2 * fl) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
        // this wave's h writes are done; after the barrier every wave's are
        wait_vm_lgkm<63, 0>();
        barrier();
        static_for<KS2 * DB>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int st = i / DB, b = i % DB;
            const bf16x8_t wv = take(std::integral_constant<int, KS1 + i>{});
#pragma unroll
            for (int f = 0; f < FT; ++f) {
                const bf16x8_t hv = *reinterpret_cast<const bf16x8_t*>(hbuf + (32 * f + tok) * kHPitch + 16 * half + 32 * st);
                acc2[b][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, hv, acc2[b][f], 0, 0, 0);
            }
        });
    }

    // ---- FC2 epilogue: token m0 + 32 f + tok, columns 32 (wave DB + b) + 8 g + 4 half .. +3 ----
#pragma unroll
    for (int f = 0; f < FT; ++f) {
        const int64_t m = m0 + 32 * f + tok;
        if (m >= p.M) continue;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * (wave * DB + b) + 8 * g + 4 * half;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc2[b][f][4 * g + e];
                if constexpr (SPL) {
                    *reinterpret_cast<f32x4_t*>(p.ws + (part * p.M + m) * D + col) = f32x4_t{v[0], v[1], v[2], v[3]};
                    continue;
                }
                if (p.b2) {
                    const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(p.b2 + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += bv[e];
                }
                const int64_t off = m * D + col;
                if (p.res) {
                    const uint2 rv = *reinterpret_cast<const uint2*>(p.res + off);
                    v[0] += __uint_as_float(rv.x << 16);
                    v[1] += __uint_as_float(rv.x & 0xFFFF0000u);
                    v[2] += __uint_as_float(rv.y << 16);
                    v[3] += __uint_as_float(rv.y & 0xFFFF0000u);
                }
                *reinterpret_cast<uint2*>(p.y + off) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
    }
}

// y = bf16(ws[0] + ... + ws[parts-1] + b2 [+ residual]), 8 columns a thread (D is a
// multiple of 256)
__global__ __launch_bounds__(256) void ffn_reduce_kernel(const FfnArgs p) {
    const int64_t groups = p.M * (p.D / 8);
    const int64_t half = p.M * p.D;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < groups;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t off = 8 * i;
        const int col = static_cast<int>(off % p.D);
        float v[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p.ws + off + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * h + e] = a[e];
        }
        for (int q = 1; q < p.parts; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p.ws + q * half + off + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * h + e] += a[e];
            }
        if (p.b2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(p.b2 + col + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * h + e] += bv[e];
            }
        }
        if (p.res) {
            const u32x4_t rv = *reinterpret_cast<const u32x4_t*>(p.res + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] += __uint_as_float(rv[e] << 16);
                v[2 * e + 1] += __uint_as_float(rv[e] & 0xFFFF0000u);
            }
        }
        *reinterpret_cast<u32x4_t*>(p.y + off) = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    }
}

template <int ACT, int FT, bool SPL>
hipError_t launch_d(const FfnArgs& a, hipStream_t s) {
    const int64_t blocks = (a.M + 32 * FT - 1) / (32 * FT) * (SPL ? a.parts : 1);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (a.D) {
        case 256: hipLaunchKernelGGL((ffn_kernel<ACT, 1, FT, SPL>), grid, dim3(512), 0, s, a); break;
        case 512: hipLaunchKernelGGL((ffn_kernel<ACT, 2, FT, SPL>), grid, dim3(512), 0, s, a); break;
        case 768: hipLaunchKernelGGL((ffn_kernel<ACT, 3, FT, SPL>), grid, dim3(512), 0, s, a); break;
        case 1024:
            if constexpr (FT == 1 && !SPL) {   // 64 tokens of 1024 columns do not fit LDS beside h; no split
                hipLaunchKernelGGL((ffn_kernel<ACT, 4, FT, SPL>), grid, dim3(512), 0, s, a);
                break;
            } else {
                return hipErrorInvalidValue;
            }
        default: return hipErrorInvalidValue;
    }
    if constexpr (SPL) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t groups = a.M * (a.D / 8);
        const int64_t rb = (groups + 255) / 256;
        hipLaunchKernelGGL(ffn_reduce_kernel, dim3(static_cast<unsigned>(rb < 2048 ? rb : 2048)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// 64 tokens per workgroup (half the weight traffic): split, from 4096 tokens (measured 1.15-
// 1.2x faster than 32 there, 0.8x at 128-2048); unsplit, from 16384 (where 64-token blocks
// still fill the CUs).  d_model 1024 always takes 32.  DLF_FFN_TOK=32|64 forces one (tests).
template <int ACT>
hipError_t launch_act(const FfnArgs& a, hipStream_t s) {
    int tok = a.M >= (a.parts > 1 ? 4096 : 64 * 256) && a.D <= 768 ? 64 : 32;
    const int t = options().ffn_tok;
    if (t == 32 || (t == 64 && a.D <= 768)) tok = t;
    if (a.parts > 1) return tok == 64 ? launch_d<ACT, 2, true>(a, s) : launch_d<ACT, 1, true>(a, s);
    return tok == 64 ? launch_d<ACT, 2, false>(a, s) : launch_d<ACT, 1, false>(a, s);
}

}  // namespace

int ffn_parts(int64_t M, int D, int F) {
    // built for d_model <= 768 (and S <= the chunks of d_ff).  Every workgroup streams its
    // part of the weights from L2 at a rate of its own CU until about 160 CUs together reach
    // the L2's rate (measured: 32 to 188 token blocks unsplit take the same 107-112 us on
    // BERT-base, 12 chunks; 256 workgroups of 6 chunks 80 us).  So: split only below 160
    // token blocks, into as many parts as fit one round of 256 workgroups.
    // The split's fp32 partial sums make a round trip through memory, 8 S M D bytes, which can
    // exceed the 4 M F bytes of h that the fusion keeps on chip (BERT-base: 9.4 MB against
    // 1.6 MB at 128 tokens and 12 parts, 100.7 MB against 100.7 MB at 8192 tokens and 2).  The
    // choice is made on time, which includes that traffic: 19.6 us against 112 us unsplit at
    // 128 tokens, 116 us against 126-153 us at 8192; from 16384 tokens the walk is unsplit.
    const int nchunks = F / kChunk;
    if (D > 768 || nchunks < 2 || M <= 0) return 1;
    const int want = options().ffn_split;
    if (want == 1) return 1;
    if (want > 1) return want < nchunks ? want : nchunks;
    if (M >= 64 * 256) return 1;
    const int64_t tok = M >= 4096 ? 64 : 32;                     // as launch_act takes for a split
    const int64_t blocks = (M + tok - 1) / tok;
    if (blocks >= 160) return 1;
    const int64_t fit = 256 / blocks;
    return static_cast<int>(fit < nchunks ? fit : nchunks);
}

hipError_t launch_ffn(const FfnArgs& a, int act, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (a.F <= 0 || a.F % kChunk != 0) return hipErrorInvalidValue;
    if (a.parts > 1 && (!a.ws || a.D > 768 || a.parts > a.F / kChunk)) return hipErrorInvalidValue;
    switch (act) {
        case kActNone: return launch_act<kActNone>(a, s);
        case kActRelu: return launch_act<kActRelu>(a, s);
        case kActGelu: return launch_act<kActGelu>(a, s);
        case kActGeluErf: return launch_act<kActGeluErf>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlf
