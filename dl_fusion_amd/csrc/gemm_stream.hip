// Streaming GEMM for memory-bound shapes: C = act(A B^T + bias [+ residual]) with a short
// reduction (K of 128 or 256), as in the 1x1 convolutions of a ResNet bottleneck (the GEMM of
// the [n h w][c_in] pixel matrix).  The work is reading A (and the residual) once and
// writing C once; the tiled kernel reaches half the HBM bandwidth there, because each
// workgroup has only its own few K slices in flight and its tiles do not overlap their loads
// with the previous tile's epilogue.
//
// Here a workgroup of four waves owns a block of 128 to 384 output columns and is persistent
// over tiles of 32 rows of A, dealt to the workgroups of its block in turn.  B's block is
// loaded once into registers (wave w holds the MFMA fragments of a quarter of the block's
// columns for all of K).  The tiles stream through an LDS ring of R slots, each holding one
// tile's A rows and, with a residual, its residual rows, by LDS-DMA buffer loads that every
// wave shares; R tiles are in flight at a time.  Per tile a wave runs K/16 x N/128 MFMAs out
// of LDS and then its epilogue, whose stores go out after the next tile's loads.  Loads past
// the last tile or row read zeros and stores past them are dropped (out-of-range buffer
// offsets), so every wave issues the same loads and stores each iteration and the
// memory-counter waits are constants.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "mma_common.h"

namespace dlf {
namespace {

constexpr int kSRows = 32;             // rows of A per tile

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// f(integral_constant<int, I>) ... f(integral_constant<int, N-1>), unrolled at compile time
template <int I, int N, class Fn>
__device__ __forceinline__ void unrolled(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        unrolled<I + 1, N>(f);
    }
}

// CPW: 32-column output blocks per wave (a workgroup's column block is N = 128 CPW wide);
// KS: 16-wide K steps (K = 16 KS); OCC: workgroups a CU (the ring takes 128 KB of LDS over
// OCC).  The output is p.N = N nblk columns wide: workgroup b owns column block cb and walks
// the row tiles gt, gt + Gt, ... (Gt workgroups a block), with the workgroups of one row tile
// on one XCD, so that all but the first read of the tile's A rows hit its L2.
// GATHER: A's row m is output pixel m = (img, ho, wo) of an unpadded 1x1 convolution with
// strides SH, SW, read from input pixel (img, SH ho, SW wo) of the NHWC input (c_in = K).
template <int CPW, int KS, int OCC, int ACT, bool RES, bool GATHER>
__global__ __launch_bounds__(256, OCC) void gemm_stream_kernel(const MmaArgs p, const int tiles) {
    constexpr int N = 128 * CPW, K = 16 * KS;
    constexpr int kSLds = 128 * 1024 / OCC;
    constexpr int ABYTES = kSRows * K * 2, RBYTES = RES ? kSRows * N * 2 : 0;
    constexpr int SLOT = ABYTES + RBYTES;
    constexpr int LPW = SLOT / 4096;                           // 1 KB loads per wave per tile
    constexpr int ALOADS = ABYTES / 1024;                      // the A part: loads 0 .. ALOADS-1
    // output rows of 256 bytes or more go out staged, as whole rows of 16-byte stores (2 CPW
    // of 1 KB per wave); with N = 128 each lane's 8-byte pieces go out directly (4 CPW a
    // wave): measured faster each way
    constexpr bool STAGED = CPW >= 2;
    constexpr int ST = STAGED ? 2 * CPW : 4 * CPW;             // stores per wave per tile
    constexpr int CA = K / 8, CR = N / 8;                      // 16-byte chunks per row
    // tiles in flight: what the ring holds, at most 8, and few enough that the loads of R-1
    // tiles and the stores of R tiles fit the 6-bit memory counter (stores count in it too)
    constexpr int R0 = kSLds / SLOT > 8 ? 8 : kSLds / SLOT;
    constexpr int R1 = (63 + LPW) / (LPW + ST);
    constexpr int R = R0 < R1 ? R0 : R1;
    static_assert(SLOT % 4096 == 0 && R >= 2, "whole kilobyte loads, two tiles in flight");
    static_assert(LPW * (R - 1) + ST * R < 64, "vmcnt range");
    static_assert(CA >= 16 && CR >= 16, "the chunk swizzle spans 16 chunks");
    static_assert(OCC * (R * SLOT + (STAGED ? kSRows * N * 2 : 0)) <= 160 * 1024, "LDS per CU");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[R * SLOT];
    // the finished tile, rows of N values (chunks swizzled like the ring's), written out as
    // whole rows with 16-byte stores
    __shared__ __attribute__((aligned(1024))) uint8_t stage[STAGED ? kSRows * N * 2 : 16];

    const int tid = static_cast<int>(threadIdx.x);
    // the wave index in a scalar register: the LDS-DMA destination (M0) must be uniform
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), half = lane >> 5, row = lane & 31;
    const int nblk = p.N / N, b = static_cast<int>(blockIdx.x);
    const int G = static_cast<int>(gridDim.x) / nblk;                // Gt: a multiple of 8
    const int cb = (b >> 3) % nblk, wg = ((b >> 3) / nblk) * 8 + (b & 7);
    const int n0 = cb * N;                                            // first output column
    const int64_t M = p.M, LD = p.N;
    const uint32_t ho = static_cast<uint32_t>(p.Ho), wo = static_cast<uint32_t>(p.Wo);
    const int64_t a_bytes = GATHER ? M / (int64_t(ho) * wo) * p.H * p.W * K * 2 : M * K * 2;
    const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(p.a, static_cast<uint32_t>(a_bytes));
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(RES ? static_cast<const void*>(p.res) : p.a,
                                                  static_cast<uint32_t>(RES ? M * LD * 2 : 0));
    const __amdgpu_buffer_rsrc_t cr = buffer_rsrc(p.c, static_cast<uint32_t>(M * LD * 2));

    // load j of this wave fills slot bytes [(wave LPW + j) KB, +1 KB): lane's 16-byte chunk
    // q = 64 (wave LPW + j) + lane sits at row q / CA, physical chunk q % CA, which holds
    // logical chunk (q % CA) ^ (row % 16) (same for the residual part with CR chunks a row).
    // Offsets are tile-independent up to the tile's first row.
    uint32_t rel[LPW];
    int lrow[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int lj = wave * LPW + j;
        if (lj < ALOADS) {
            const int q = 64 * lj + lane, r = q / CA, pc = q % CA;
            lrow[j] = r;
            rel[j] = static_cast<uint32_t>(((GATHER ? 0 : r * K) + 8 * (pc ^ (r & 15))) * 2);
        } else {
            const int q = 64 * (lj - ALOADS) + lane, r = q / CR, pc = q % CR;
            lrow[j] = r;
            rel[j] = static_cast<uint32_t>((r * LD + n0 + 8 * (pc ^ (r & 15))) * 2);
        }
    }
    auto issue = [&](int i) {   // the loads of this workgroup's tile i into slot i % R
        const int t = wg + G * i;
        uint8_t* const slot = ring + (i % R) * SLOT;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int lj = wave * LPW + j;
            const int64_t m = static_cast<int64_t>(t) * kSRows + lrow[j];
            const bool ok = t < tiles && m < M;
            if (lj < ALOADS) {
                uint32_t off;
                if constexpr (GATHER) {
                    const uint32_t mm = static_cast<uint32_t>(m), q = mm / wo, x = mm - q * wo;
                    const uint32_t img = q / ho, y = q - img * ho;
                    const uint32_t pix = (img * static_cast<uint32_t>(p.H) + y * static_cast<uint32_t>(p.SH)) *
                                             static_cast<uint32_t>(p.W) + x * static_cast<uint32_t>(p.SW);
                    off = pix * static_cast<uint32_t>(K * 2) + rel[j];
                } else {
                    off = static_cast<uint32_t>(static_cast<int64_t>(t) * kSRows * K * 2) + rel[j];
                }
                load_lds16_buf(ar, ok ? off : kOutOfRange, slot + lj * 1024);
            } else {
                const uint32_t off = static_cast<uint32_t>(static_cast<int64_t>(t) * kSRows * LD * 2) + rel[j];
                load_lds16_buf(rr, ok ? off : kOutOfRange, slot + lj * 1024);
            }
        }
    };

    const int iters = wg < tiles ? (tiles - wg + G - 1) / G : 0;
    // the first tile's loads go out ahead of B and the bias, the other R-1 tiles' behind them:
    // B's latency overlaps the first tile's, and the wait for tile 0 below covers B too
    issue(0);
    // B fragments of this wave's columns 32 (CPW wave + j) + lane % 32, chunk 2 s + half
    bf16x8_t bf[CPW][KS];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const uint16_t* const brow = static_cast<const uint16_t*>(p.b) +
                                     static_cast<int64_t>(n0 + 32 * (CPW * wave + j) + row) * K + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) bf[j][s] = *reinterpret_cast<const bf16x8_t*>(brow + 16 * s);
    }

    // bias of this lane's output columns 32 (CPW wave + j) + 8 g + 4 half .. +3
    f32x4_t bias[CPW][4];
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bias[j][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (p.shift) bias[j][g] = *reinterpret_cast<const f32x4_t*>(p.shift + n0 + 32 * (CPW * wave + j) + 8 * g + 4 * half);
        }

#pragma unroll
    for (int i = 1; i < R; ++i) issue(i);
    for (int i = 0; i < iters; ++i) {
        // tile i has landed for this wave once at most the memory operations issued after its
        // loads are outstanding: the loads of tiles i+1 .. i+R-1 and the stores of tiles
        // max(0, i-R) .. i-1 (the stores of tile k go out right after the loads of tile k+R)
        if (i >= R) {
            wait_vmcnt<LPW * (R - 1) + ST * R>();
        } else {
            unrolled<0, R>([&](auto c) {
                if (i == decltype(c)::value) wait_vmcnt<LPW * (R - 1) + ST * decltype(c)::value>();
            });
        }
        barrier();
        const uint8_t* const slot = ring + (i % R) * SLOT;
        f32x16_t acc[CPW];
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8_t av =
                *reinterpret_cast<const bf16x8_t*>(slot + row * K * 2 + 16 * ((2 * s + half) ^ (row & 15)));
#pragma unroll
            for (int j = 0; j < CPW; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j][s], av, acc[j], 0, 0, 0);
        }
        // the residual of this lane's outputs, out of the slot before it is refilled
        uint2 rv[CPW][4];
        if constexpr (RES) {
#pragma unroll
            for (int j = 0; j < CPW; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = 32 * (CPW * wave + j) + 8 * g + 4 * half;   // 4 columns: half a chunk
                    rv[j][g] = *reinterpret_cast<const uint2*>(slot + ABYTES + row * N * 2 +
                                                              16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7));
                }
        }
        // epilogue: row lane % 32 of the tile, columns as the bias, bf16
        u32x2_t outv[CPW][4];
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[j][4 * g + e] + bias[j][g][e];
                if constexpr (RES) {
                    v[0] += __uint_as_float(rv[j][g].x << 16);
                    v[1] += __uint_as_float(rv[j][g].x & 0xFFFF0000u);
                    v[2] += __uint_as_float(rv[j][g].y << 16);
                    v[3] += __uint_as_float(rv[j][g].y & 0xFFFF0000u);
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
                outv[j][g] = u32x2_t{lo, hi};
                if constexpr (STAGED) {
                    const int col = 32 * (CPW * wave + j) + 8 * g + 4 * half;
                    *reinterpret_cast<u32x2_t*>(stage + row * N * 2 + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7)) =
                        outv[j][g];
                }
            }
        wait_vm_lgkm<63, 0>();   // this wave's slot reads (and staging writes) are done
        barrier();               // and every wave's: the slot takes tile i + R (the tile is staged)
        issue(i + R);
        const int64_t t0 = static_cast<int64_t>(wg + G * i) * kSRows;
        if constexpr (STAGED) {
            // wave w writes rows 8 w .. 8 w + 7 of the tile, 1 KB (1024 / (2 N) rows) a store,
            // whole rows of the column block: these stores write through to device scope
            // (2% on a ResNet stage's 1x1 layers); the 8-byte stores below do not (slower)
#pragma unroll
            for (int u = 0; u < ST; ++u) {
                const int q = 64 * u + lane, r = 8 * wave + q / CR, c = q % CR;
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * N * 2 + 16 * (c ^ (r & 15)));
                const int64_t m = t0 + r;
                const uint32_t off = m < M ? static_cast<uint32_t>((m * LD + n0 + 8 * c) * 2) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b128(v, cr, off, 0, kStoreDevice);
            }
        } else {
            const int64_t m = t0 + row;
#pragma unroll
            for (int j = 0; j < CPW; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = 32 * (CPW * wave + j) + 8 * g + 4 * half;
                    const uint32_t off = m < M ? static_cast<uint32_t>((m * LD + n0 + col) * 2) : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b64(outv[j][g], cr, off, 0, 0);
                }
        }
    }
    wait_vmcnt<0>();   // the dummy loads of the ring's last slots land before the workgroup ends
}

template <int CPW, int KS, int OCC, int ACT>
hipError_t launch3(const MmaArgs& a, int tiles, hipStream_t s) {
    // Gt workgroups a column block, a multiple of 8 (the tile-to-XCD mapping), at most the
    // CUs' OCC slots
    const int nblk = a.N / (128 * CPW);
    const int cap = (256 * OCC / nblk) / 8 * 8, want = (tiles + 7) / 8 * 8;
    const dim3 grid(static_cast<unsigned>((want < cap ? want : cap) * nblk));
    if (a.Wo > 0)   // the strided 1x1 convolution: no residual (gemm_stream_ok)
        hipLaunchKernelGGL((gemm_stream_kernel<CPW, KS, OCC, ACT, false, true>), grid, dim3(256), 0, s, a, tiles);
    else if (a.res)
        hipLaunchKernelGGL((gemm_stream_kernel<CPW, KS, OCC, ACT, true, false>), grid, dim3(256), 0, s, a, tiles);
    else
        hipLaunchKernelGGL((gemm_stream_kernel<CPW, KS, OCC, ACT, false, false>), grid, dim3(256), 0, s, a, tiles);
    return hipGetLastError();
}

template <int CPW, int KS, int OCC>
hipError_t launch2(const MmaArgs& a, int act, int tiles, hipStream_t s) {
    switch (act) {
        case kActNone: return launch3<CPW, KS, OCC, kActNone>(a, tiles, s);
        case kActRelu: return launch3<CPW, KS, OCC, kActRelu>(a, tiles, s);
        case kActGelu: return launch3<CPW, KS, OCC, kActGelu>(a, tiles, s);
        case kActGeluErf: return launch3<CPW, KS, OCC, kActGeluErf>(a, tiles, s);
        default: return hipErrorInvalidValue;
    }
}

// built column blocks: 128, 256 and 384 wide for K = 128, 128 and 256 for K = 256 (B's
// fragments take N K / 512 registers a lane, at most 128)
bool built(int64_t nb, int64_t k) { return (k == 128 && nb <= 384) || (k == 256 && nb <= 256); }

// a workgroup's column block: the widest built one that divides N (128 for gathered rows:
// measured 1.2x faster than 256 on the strided 1x1 56x56x256 -> 28x28x512, where B's 128 KB
// a workgroup cost more than the fourfold reads of A), or what DLF_STREAM_NB asks for where
// that is built and divides N (tuning only); 0 if none
int64_t block_cols(int64_t n, int64_t k, bool gather) {
    const int64_t nb = options().stream_nb;
    if (nb != 0 && n % nb == 0 && built(nb, k)) return nb;
    if (gather) return n % 128 == 0 ? 128 : 0;
    for (const int64_t nb : {384, 256, 128})
        if (n % nb == 0 && built(nb, k)) return nb;
    return 0;
}

}  // namespace

bool gemm_stream_ok(const MmaArgs& a) {
    if (a.scale || a.parts > 1 || a.M <= 0 || a.N <= 0) return false;
    if (a.K != 128 && a.K != 256) return false;
    const int64_t nb = block_cols(a.N, a.K, a.Wo > 0);
    if (nb == 0 || a.N / nb > 32) return false;                   // at least 8 workgroups a block
    const int64_t lim = int64_t(1) << 31;
    if (a.Wo > 0) {   // gathered rows: an unpadded 1x1 convolution, without residual
        if (a.res || a.KW != 1 || a.PH != 0 || a.PW != 0 || a.Cin != a.K || a.Ho <= 0 || a.SH <= 0 || a.SW <= 0)
            return false;
        const int64_t px = int64_t(a.Ho) * a.Wo;
        if (a.M % px != 0 || int64_t(a.SH) * (a.Ho - 1) >= a.H || int64_t(a.SW) * (a.Wo - 1) >= a.W) return false;
        if (a.M / px * a.H * a.W * a.K * 2 >= lim) return false;
    }
    return a.M * a.K * 2 < lim && a.M * a.N * 2 < lim;
}

bool gemm_stream_pays(const MmaArgs& a) {
    // measured on MI355X against the tiled kernel: 1.1-1.4x faster from 4M outputs with
    // N = 128 to 384 (32768 rows of 128, 25088 rows of 256 or 384), 1.1-2.2x with N = 512 to
    // 1024 in column blocks, 0.97x at 25088 rows of 128.  A variant with B blocks of K = 512
    // (and so N = 128) was slower and is not built.
    // Gathered rows (strided 1x1 convolutions) pay from N = 512 only: 1.23x at 56x56x256 ->
    // 28x28x512 (stride 2), 0.75x at 56x56x256 -> 28x28x256, where the implicit GEMM's
    // tiles read the strided rows faster.
    if (a.Wo > 0 && a.N < 512) return false;
    return gemm_stream_ok(a) && a.M * a.N >= (int64_t(1) << 22);
}

hipError_t launch_gemm_stream(const MmaArgs& a, int act, hipStream_t s) {
    const int64_t tiles64 = (a.M + kSRows - 1) / kSRows;
    const int tiles = static_cast<int>(tiles64);
    const int64_t nb = block_cols(a.N, a.K, a.Wo > 0);
    const int cpw = static_cast<int>(nb / 128), ks = static_cast<int>(a.K / 16);
    // two workgroups a CU (half the ring each) where the block's N K = 32768, from 2048 units
    // of a row tile and a column block: measured 1.05-1.2x faster there, 0.95x at 1250.  With
    // N = K = 128 two were level to 4% slower; N = 384 has no room for two (its staging
    // area), and N = K = 256 needs more than 256 registers for its B fragments and
    // accumulators.
    const bool two = cpw * ks == 16 && tiles64 * (a.N / nb) >= 2048;
    switch (cpw * 1000 + ks * 10 + (two ? 2 : 1)) {
        case 1081: return launch2<1, 8, 1>(a, act, tiles, s);
        case 1161: return launch2<1, 16, 1>(a, act, tiles, s);
        case 1162: return launch2<1, 16, 2>(a, act, tiles, s);
        case 2081: return launch2<2, 8, 1>(a, act, tiles, s);
        case 2082: return launch2<2, 8, 2>(a, act, tiles, s);
        case 2161: return launch2<2, 16, 1>(a, act, tiles, s);
        case 3081: return launch2<3, 8, 1>(a, act, tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlf
