// Stride-1 3x3 convolution (bf16, pad 1) as an implicit GEMM whose activation
// operand never leaves LDS: the fused Conv -> BN -> [residual] -> act kernel for
// the ResNet-stage shapes.
//
// A workgroup (4 waves) owns TH output rows x the full width of one image and
// 64 output channels.  It loads the (TH+2) x (W+2) x Cin input halo (zero
// outside the image) into LDS once, straight from global memory, and builds the
// A fragments of all nine taps from it by shifted reads; there is no per-tap
// re-fetch of the input, which is what makes the generic implicit GEMM fetch
// every input pixel nine times.  The folded weights W' (OHWI, i.e. [co][tap][ci])
// stream through a four-stage LDS ring in slices of one tap x 64 input channels,
// with the same software pipeline as the GEMM kernel: fragment double buffering,
// LDS reads interleaved with the MFMAs, one barrier per slice, refills issued
// S slices ahead.  The contraction is v_mfma_f32_32x32x16_bf16 issued as
// D = W . X^T, so a lane holds one output pixel and runs of four consecutive
// output channels; the epilogue (bias, residual, activation, one rounding) runs
// on those registers and the tile leaves through LDS with coalesced 16-byte
// stores, each output element written once: the conv + epilogue of
// "OpenPPL算子融合深度解析" §4.3, with the zero padding of the direct
// convolution loop in the discosf.com fusion article §3.3.
//
// LDS layouts (16-byte chunks XOR-swizzled so that the 16 lanes one fragment
// read serves per cycle hit 16 distinct bank groups):
//   halo:   pixel-major, Cin*2 bytes per pixel; chunk k of pixel q is stored at
//           k ^ ((q >> 1) & 7) when Cin == 64, k ^ (q & 15) when Cin >= 128.
//   weights: 64 rows (output channels) x 128 bytes; chunk k of row r at k ^ ((r >> 1) & 7).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "mma_common.h"

namespace dlf {
namespace {

constexpr int kCo = 64;                    // output channels per workgroup
constexpr int kS = 4;                      // weight ring stages
constexpr int kWStage = kCo * 128;         // one weight slice: 64 rows x 128 bytes
constexpr int kWLoads = kWStage / 1024 / 4;   // 1 KB weight loads per wave per slice (2)

__device__ __forceinline__ int wchunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Chunk swizzle of halo pixel (hr, wc) of an image of width W, keyed on its unpadded index
// hr * W + wc - 1: the output pixels a fragment read serves are consecutive in that index even
// across a row end (where the halo index jumps by 2), so 16 of them always take 16 distinct
// (pixel parity, chunk position) bank slots.
__device__ __forceinline__ int hswz(int hr, int wc, int W) { return ((hr * W + wc - 1) >> 1) & 7; }

// Output staging: 64 channels = 128 B per pixel row; chunk c of row m sits at
// c ^ ((m >> 1) & 7), so the 32 rows one 8-byte register write covers fall on
// 16 distinct (row parity, chunk) slots and the 16-byte read-back of two
// neighbouring rows by 16 lanes touches every bank group once.
__device__ __forceinline__ int stg_swz(int m) { return (m >> 1) & 7; }

template <int WF, int HALO_KB, int ACT>
__global__ __launch_bounds__(256, 1) void conv_halo_kernel(const HaloArgs p, const int th, const int row_tiles) {
    constexpr int HALO = HALO_KB * 1024;
    constexpr int STAGED = 4 * WF * 32 * kCo * 2;          // output tile staging (reuses the LDS)
    constexpr int RING = kS * kWStage;
    constexpr int SMEM = HALO + RING > STAGED ? HALO + RING : STAGED;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    uint8_t* const halo = smem;
    uint8_t* const ring = smem + HALO;

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    // workgroup -> (co tile, image, row tile); consecutive ids share an image (L2 reuse)
    const int bid = static_cast<int>(blockIdx.x);
    const int co_tile = bid % p.co_tiles;
    const int rt_img = bid / p.co_tiles;
    const int img = rt_img / row_tiles, rt = rt_img - img * row_tiles;
    const int h0 = rt * th;
    const int th_eff = min(th, p.H - h0);
    const int W = p.W, W2 = p.W + 2, Cin = p.Cin;
    const int npix = th_eff * W;                            // output pixels of this tile
    const int c0 = co_tile * kCo;
    const int K = 9 * Cin;
    const int Q = Cin >> 6;                                 // 64-channel groups
    const int KT = 9 * Q;                                   // K slices
    const int ps = Cin * 2;                                 // halo bytes per pixel
    const int sh = Cin >= 128 ? 0 : 1, xm = Cin >= 128 ? 15 : 7;   // halo swizzle
    // this image and this tile's 64 weight rows as buffers (the host keeps an image below 2 GB):
    // the loads are then not FLAT instructions, so the compiler counts outstanding LDS reads
    // exactly instead of waiting for every one (and every load in flight) before each MFMA;
    // positions outside the image and slices past the last read zeros
    const __amdgpu_buffer_rsrc_t xr =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.x) + static_cast<int64_t>(img) * p.H * W * ps,
                    static_cast<uint32_t>(p.H * W * ps));
    const __amdgpu_buffer_rsrc_t wr_ =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.w) + static_cast<int64_t>(c0) * K * 2, static_cast<uint32_t>(kCo * K * 2));

    // ---- halo: (th+2) x (W+2) pixels, one 1 KB load instruction per 1024/ps pixels ----
    {
        const int nhp = (th_eff + 2) * W2;
        const int nhi = (nhp * ps + 1023) >> 10;
        for (int li = wave; li < nhi; li += 4) {
            const int byte = li * 1024 + lane * 16;
            const int q = byte / ps, pc = (byte - q * ps) >> 4;
            const int lc = pc ^ ((q >> sh) & xm);
            const int hr = q / W2, wc = q - hr * W2;
            const int hi = h0 - 1 + hr, wi = wc - 1;
            const bool ok = q < nhp && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                            static_cast<unsigned>(wi) < static_cast<unsigned>(W);
            const uint32_t off = static_cast<uint32_t>((hi * W + wi) * ps + lc * 16);
            load_lds16_buf(xr, ok ? off : kOutOfRange, halo + li * 1024);
        }
    }

    // ---- weight slices: slice kt = (tap kt / Q, channel group kt % Q); past KT: zeros ----
    auto issue_w = [&](int kt) {
        uint8_t* st = ring + (kt % kS) * kWStage;
        const bool kin = kt < KT;
        const int t = kin ? kt / Q : 0, q = kin ? kt - (kt / Q) * Q : 0;
#pragma unroll
        for (int j = 0; j < kWLoads; ++j) {
            const int blk = wave * kWLoads + j;                 // 8 rows per 1 KB
            const int r = blk * 8 + (lane >> 3), pc = lane & 7;
            const int lc = wchunk(r, pc);
            const uint32_t off = static_cast<uint32_t>((r * K + t * Cin + q * 64 + lc * 8) * 2);
            load_lds16_buf(wr_, kin ? off : kOutOfRange, st + blk * 1024);
        }
    };

    // ---- this lane's pixels: fragment i holds tile pixel (wave*WF + i)*32 + (lane & 31) ----
    int hp[WF];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int pix = (wave * WF + i) * 32 + (lane & 31);
        const int pp = pix < npix ? pix : 0;
        const int ho = pp / W;
        hp[i] = ho * W2 + (pp - ho * W);                    // halo pixel of tap (0, 0)
    }

    f32x16_t acc[2][WF];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < WF; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    bf16x8_t xf[2][WF], wf[2][2];
    auto read_frags = [&](auto b_c, int kt, int st) {
        constexpr int b = decltype(b_c)::value;
        const int t = kt / Q, q = kt - t * Q;
        const int r = t / 3, s = t - r * 3;
        const int c = 2 * st + (lane >> 5);                 // 16-byte chunk within the 64 channels
        const int cix = q * 8 + c;
#pragma unroll
        for (int i = 0; i < WF; ++i) {
            const int qp = hp[i] + r * W2 + s;
            xf[b][i] = *reinterpret_cast<const bf16x8_t*>(halo + qp * ps + ((cix ^ ((qp >> sh) & xm)) << 4));
        }
        const uint8_t* stg = ring + (kt % kS) * kWStage;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 32 * j + (lane & 31);
            wf[b][j] = *reinterpret_cast<const bf16x8_t*>(stg + row * 128 + (wchunk(row, c) << 4));
        }
    };
    auto mma_all = [&](auto b_c) {
        constexpr int b = decltype(b_c)::value;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < WF; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b][j], xf[b][i], acc[j][i], 0, 0, 0);
    };
    constexpr int MF = 2 * WF, R = 2 + WF;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

#pragma unroll
    for (int s2 = 0; s2 < kS; ++s2) issue_w(s2);
    wait_vmcnt<(kS - 1) * kWLoads>();   // the halo and weight slice 0 have landed
    barrier();
    read_frags(I0{}, 0, 0);

    // four k-steps of 16 channels per slice; the transition to slice kt+1 happens in step 3
    for (int kt = 0; kt < KT; ++kt) {
        read_frags(I1{}, kt, 1);
        mma_all(I0{});
        interleave<MF, R, 0>();
        read_frags(I0{}, kt, 2);
        mma_all(I1{});
        interleave<MF, R, 0>();
        read_frags(I1{}, kt, 3);
        mma_all(I0{});
        interleave<MF, R, 0>();
        wait_vmcnt<(kS - 2) * kWLoads>();
        barrier();
        issue_w(kt + kS);
        read_frags(I0{}, kt + 1 < KT ? kt + 1 : kt, 0);
        mma_all(I1{});
        interleave<MF, R, kWLoads>();
    }

    wait_vmcnt<0>();   // the zero-page refills past the last slice have landed
    // ---- epilogue: lane holds pixel (wave*WF + i)*32 + (lane & 31) and, in register group g,
    //      output channels 32 j + 8 g + 4 (lane / 32) + e%4 of this tile ----
    __syncthreads();   // the LDS is reused for staging
    const int lrow = lane & 31, half = lane >> 5;
    constexpr int SROW = kCo * 2, CPR = SROW / 16;
    const int64_t m0 = (static_cast<int64_t>(img) * p.H + h0) * W;   // first output row of the tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = 32 * j + 8 * g + 4 * half;
            float sh4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) {
                const f32x4_t t = *reinterpret_cast<const f32x4_t*>(p.bias + c0 + nl);
                sh4[0] = t[0]; sh4[1] = t[1]; sh4[2] = t[2]; sh4[3] = t[3];
            }
#pragma unroll
            for (int i = 0; i < WF; ++i) {
                const int ml = (wave * WF + i) * 32 + lrow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * g + e] + sh4[e];
                if (p.res) {
                    const int64_t mr = m0 + (ml < npix ? ml : 0);
                    const uint2 t = *reinterpret_cast<const uint2*>(p.res + mr * p.Cout + c0 + nl);
                    v[0] += __uint_as_float(t.x << 16);
                    v[1] += __uint_as_float(t.x & 0xFFFF0000u);
                    v[2] += __uint_as_float(t.y << 16);
                    v[3] += __uint_as_float(t.y & 0xFFFF0000u);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = activate<ACT>(v[e]);
                const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                                    (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
                const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(v[2])) |
                                    (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
                const int cb = nl * 2;
                *reinterpret_cast<uint2*>(smem + ml * SROW + (((cb >> 4) ^ stg_swz(ml)) << 4) + (cb & 15)) =
                    make_uint2(lo, hi);
            }
        }
    }
    __syncthreads();
    uint8_t* const yb = reinterpret_cast<uint8_t*>(p.y);
    for (int qd = tid; qd < npix * CPR; qd += 256) {
        const int ml = qd / CPR, cc = qd - ml * CPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + ml * SROW + ((cc ^ stg_swz(ml)) << 4));
        *reinterpret_cast<u32x4_t*>(yb + ((m0 + ml) * p.Cout + c0) * 2 + cc * 16) = v;
    }
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// ---- 64 input channels: weights resident in LDS, persistent workgroups ----
//
// With Cin = 64 all nine taps of a 64-channel output tile are 72 KB, so each
// workgroup loads them once and keeps them; the rest of LDS holds two halo
// buffers.  One workgroup per CU walks a list of row tiles.  Its eight waves are
// split by role: four consumer waves (one per SIMD) only read LDS, issue MFMAs
// and run the register epilogue into LDS staging; four producer waves own all
// global memory traffic: the next tile's halo (LDS-DMA into the idle buffer) and
// the previous tile's output (read back from staging, written as whole 128-byte
// rows).  A producer stalled on memory never holds up the matrix pipe of its
// SIMD.  Tiles are dealt to the eight XCDs in contiguous ranges (workgroup b runs
// on XCD b mod 8), so the halo rows that neighbouring tiles share are fetched
// once per L2.
//
// Per tile k (halo buffer b = k mod 2), both roles pass the same two barriers:
//   consumers: compute on b | Y_k | epilogue into staging (reusing b) | X_k+1
//   producers: store tile k-1 from staging in b^1, load halo k+1 into b^1,
//              wait for both                          | Y_k |              | X_k+1
// The first tile has one more, X_0': X_0 publishes the first halo and weight taps
// 0..2, X_0' (before the consumers read tap 3) taps 3..8, so the MFMAs of the first
// twelve k-steps overlap the rest of the weight fill.
// Producer wave w reads back, and later loads the halo into, only the 1 KB
// blocks w, w + 4, w + 8, ... of a buffer, so its own LDS reads are the only
// ones that must finish before its halo loads reuse the space.
//
// Every address that does not change from tile to tile is computed once: the
// consumer's fragment reads cost one XOR each, the producer's halo loads a
// select and a compare each.
constexpr int kRWeights = 9 * kWStage;   // 72 KB
constexpr int kRHalo = 44 * 1024;        // one halo buffer: (th + 2) (W + 2) pixels x 128 B
constexpr int kRLoads = kRHalo / 4096;   // halo loads per producer wave (1 KB each)
constexpr int kRBlocks = 256;            // 32 per XCD
constexpr int kRDist = 3;                // fragment prefetch distance (k-steps)

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0) only

template <int WF, int ACT>
__global__ __launch_bounds__(512, 1) void conv_halo_res_kernel(const HaloArgs p, const int th, const int row_tiles,
                                                               const int per_xcd) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kRWeights + 2 * kRHalo];
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int bid = static_cast<int>(blockIdx.x);
    const int xcd = bid & 7, jb = bid >> 3;
    const int co_tile = jb % p.co_tiles, U = 32 / p.co_tiles;
    const int T = p.N * row_tiles;
    const int s_end = min(T, (xcd + 1) * per_xcd);
    const int s_first = xcd * per_xcd + jb / p.co_tiles;
    if (s_first >= s_end) return;
    const int W = p.W, W2 = p.W + 2, H = p.H;
    const int c0 = co_tile * kCo;
    constexpr int SROW = kCo * 2;

    if (wave >= 4) {
        // ================= producers =================
        const int pw = wave - 4, ptid = tid - 256;
        const uint8_t* const xb = reinterpret_cast<const uint8_t*>(p.x);
        const uint8_t* const wb = reinterpret_cast<const uint8_t*>(p.w);
        uint8_t* const yb = reinterpret_cast<uint8_t*>(p.y);
        // weights of this output tile: tap t at smem + t * 8 KB, 64 rows x 128 B, swizzled chunks;
        // load l = pw + 4 n is tap l / 8, rows 8 (l % 8) .. +7, and l % 8 is pw or pw + 4.  Loads
        // 0..5 (taps 0..2) go out first, before any halo address is computed, loads 6..17 (taps
        // 3..8) after the first halo: the first tile starts once taps 0..2 and its halo are in.
        // (all loads use the buffer form: the 64 weight rows and each tile's image as buffers,
        // with halo positions outside the image at an offset past the end, which reads zeros)
        const int wr0 = pw * 8 + (lane >> 3), wr1 = wr0 + 32;
        const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(wb + static_cast<int64_t>(c0) * 576 * 2, 64 * 576 * 2);
        const uint32_t w0 = static_cast<uint32_t>((wr0 * 576 + wchunk(wr0, lane & 7) * 8) * 2);
        const uint32_t w1 = static_cast<uint32_t>((wr1 * 576 + wchunk(wr1, lane & 7) * 8) * 2);
        auto load_weights = [&](auto n0_c, auto n1_c) {
            static_for<decltype(n0_c)::value, decltype(n1_c)::value>([&](auto n_c) {
                constexpr int n = decltype(n_c)::value;
                const int l = pw + 4 * n, tap = l >> 3;
                load_lds16_buf(wrs, ((l & 7) < 4 ? w0 : w1) + tap * 128, smem + tap * kWStage + (l & 7) * 1024);
            });
        };
        load_weights(std::integral_constant<int, 0>{}, std::integral_constant<int, 6>{});
        // halo load n of this wave covers halo pixel q_n = 8 (pw + 4 n) + lane / 8, chunk lane % 8
        // (stored at swizzled chunk position lane % 8, i.e. global chunk lc_n).  Tile-independent:
        // the byte offset from halo pixel (0, 0), the halo row, and whether the column is inside.
        // q / W2 is taken as (q + 1/2) / W2 in fp32: exact for q < 2^12 and W2 <= 258, since the
        // product is never within 1/(2 W2) of an integer while its rounding error stays below 1e-3.
        const float rw2 = 1.0f / static_cast<float>(W2);
        int voff[kRLoads], hrow[kRLoads];
        uint32_t colok = 0;
#pragma unroll
        for (int n = 0; n < kRLoads; ++n) {
            const int q = 8 * (pw + 4 * n) + (lane >> 3);
            const int hr = static_cast<int>((static_cast<float>(q) + 0.5f) * rw2), wc = q - hr * W2;
            hrow[n] = hr;
            voff[n] = (hr * W + wc - 1) * 128 + (((lane & 7) ^ ((q >> 1) & 7)) << 4);
            if (wc >= 1 && wc <= W) colok |= 1u << n;
        }
        // halo of spatial tile st into buf (zero outside the image)
        auto load_halo = [&](int st, uint8_t* buf) {
            const int img = st / row_tiles, h0 = (st - img * row_tiles) * th;
            const int the = min(th, H - h0);
            const int nhp = (the + 2) * W2;
            const int nhi = (nhp * 128 + 1023) >> 10;
            // rows of the halo inside the image: hr in [rlo, rhi)
            const int rlo = h0 == 0 ? 1 : 0, rhi = min(the + 2, H - h0 + 1);
            const __amdgpu_buffer_rsrc_t xr =
                buffer_rsrc(xb + static_cast<int64_t>(img) * H * W * 128, static_cast<uint32_t>(H * W * 128));
            const int row0 = (h0 - 1) * W * 128;   // halo pixel (0, 0) sits one row above h0
            const int q0 = 8 * pw + (lane >> 3);
#pragma unroll
            for (int n = 0; n < kRLoads; ++n) {
                if (pw + 4 * n >= nhi) break;
                const bool ok = ((colok >> n) & 1u) && q0 + 32 * n < nhp && hrow[n] >= rlo && hrow[n] < rhi;
                load_lds16_buf(xr, ok ? static_cast<uint32_t>(row0 + voff[n]) : kOutOfRange, buf + (pw + 4 * n) * 1024);
            }
        };
        // staged output of spatial tile st (in buf) -> y; lane handles chunk ptid % 8 of rows
        // ptid / 8 + 32 i, so both addresses advance by constants (the swizzle repeats every 16
        // rows).  Eight lanes write a whole 128-byte line, so the stores write through to device
        // scope.
        auto store_tile = [&](int st, const uint8_t* buf) {
            const int img = st / row_tiles, h0 = (st - img * row_tiles) * th;
            const int npix = min(th, H - h0) * W;
            const int ml0 = ptid >> 3, cc = ptid & 7;
            const uint8_t* src = buf + ml0 * SROW + ((cc ^ stg_swz(ml0)) << 4);
            const __amdgpu_buffer_rsrc_t yr =
                buffer_rsrc(yb + ((static_cast<int64_t>(img) * H + h0) * W * p.Cout + c0) * 2,
                            static_cast<uint32_t>(npix * p.Cout * 2));
            uint32_t voff = static_cast<uint32_t>(ml0 * p.Cout * 2 + cc * 16);
            const uint32_t dstep = static_cast<uint32_t>(32 * p.Cout * 2);
            for (int ml = ml0; ml < npix; ml += 32, src += 32 * SROW, voff += dstep)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(src), yr, voff, 0,
                                                       kStoreDevice);
        };
        load_halo(s_first, smem + kRWeights);
        load_weights(std::integral_constant<int, 6>{}, std::integral_constant<int, 18>{});
        wait_vmcnt<12>();   // all but the twelve loads of taps 3..8
        barrier();   // X_0
        wait_vmcnt<0>();
        barrier();   // X_0': taps 3..8
        int k = 0;
        for (int s = s_first; s < s_end; s += U, ++k) {
            uint8_t* const other = smem + kRWeights + ((k + 1) & 1) * kRHalo;
            if (k > 0) store_tile(s - U, other);
            wait_lgkm0();   // this wave's staging reads are done before its halo loads reuse the blocks
            if (s + U < s_end) load_halo(s + U, other);
            wait_vmcnt<0>();
            barrier();   // Y_k
            barrier();   // X_k+1
        }
        store_tile(s_first + (k - 1) * U, smem + kRWeights + ((k - 1) & 1) * kRHalo);
        return;
    }

    // ================= consumers =================
    const int tp = th * W;
    const int half = lane >> 5;
    // x fragment of tap t: halo pixel qp = hq + (t / 3) W2 + t % 3 of this lane's output pixel;
    // chunk c sits at (qp 128 + swizzle(qp) 16) ^ (c << 4), and c = 2 st + half, so the address
    // of k-step (t, st) is xa[i][t] ^ (32 st) with half folded into xa.
    int xa[WF][9];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int pix = (wave * WF + i) * 32 + (lane & 31);
        const int pp = pix < tp ? pix : 0;
        const int ho = pp / W;
        const int hq = ho * W2 + (pp - ho * W);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int qp = hq + (t / 3) * W2 + t % 3;
            xa[i][t] = (qp * 128 + (((qp >> 1) & 7) << 4)) ^ (half << 4);
        }
    }
    // weight row 32 j + lane % 32, chunk 2 st + half of tap t at t * 8 KB + woff[j][st]
    int woff[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 32 * j + (lane & 31);
#pragma unroll
        for (int st = 0; st < 4; ++st) woff[j][st] = row * 128 + (((2 * st + half) ^ ((row >> 1) & 7)) << 4);
    }
    // bias in the accumulator layout: register 4g + e of set j holds channel 32j + 8g + 4 half + e;
    // it enters the first MFMA as its C operand, so the epilogue needs no add
    f32x16_t biasv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4_t b4 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) b4 = *reinterpret_cast<const f32x4_t*>(p.bias + c0 + 32 * j + 8 * g + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) biasv[j][4 * g + e] = b4[e];
        }
    // staging address of chunk 0 of each fragment row (with this lane's half); chunk c is
    // sbase ^ (c << 4) because the swizzle occupies address bits 4..6
    int sbase[WF];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int ml = (wave * WF + i) * 32 + (lane & 31);
        sbase[i] = ml * SROW + (stg_swz(ml) << 4) + 8 * half;
    }
    barrier();   // X_0
    int k = 0;
    for (int s = s_first; s < s_end; s += U, ++k) {
        uint8_t* const hb = smem + kRWeights + (k & 1) * kRHalo;
        const int hoff = (k & 1) * kRHalo;   // hb - halo buffer 0; a multiple of 1 KB

        // ---- 36 k-steps (9 taps x 4 x 16 channels), fragments read kRDist steps ahead ----
        f32x16_t acc[2][WF];
        bf16x8_t xf[4][WF], wf[4][2];
        auto rd = [&](auto g_c) {
            constexpr int g = decltype(g_c)::value;
            constexpr int t = g >> 2, st = g & 3, b = g & 3;
#pragma unroll
            for (int i = 0; i < WF; ++i)
                xf[b][i] = *reinterpret_cast<const bf16x8_t*>(smem + kRWeights + ((hoff + xa[i][t]) ^ (32 * st)));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                wf[b][j] = *reinterpret_cast<const bf16x8_t*>(smem + t * kWStage + woff[j][st]);
        };
        static_for<0, kRDist>(rd);
        static_for<0, 36>([&](auto g_c) {
            constexpr int g = decltype(g_c)::value;
            constexpr int b = g & 3;
            // first tile: taps 3..8 of the weights are known to have landed only after X_0'
            if constexpr (g + kRDist == 12) {
                if (k == 0) barrier();   // X_0'
            }
            if constexpr (g + kRDist < 36) rd(std::integral_constant<int, g + kRDist>{});
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < WF; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b][j], xf[b][i],
                                                                        g == 0 ? biasv[j] : acc[j][i], 0, 0, 0);
            // keep the program order: this step's MFMAs consume reads issued kRDist steps earlier
            __builtin_amdgcn_sched_barrier(0);
        });
        barrier();   // Y_k: every consumer is done with this halo; the next one has landed

        // ---- epilogue (bias is already in acc): residual, activation, one rounding, staged in hb ----
        auto stage = [&](auto res_c) {
            constexpr bool RES = decltype(res_c)::value;
            const int img = s / row_tiles, h0 = (s - img * row_tiles) * th;
            const int npix = min(th, H - h0) * W;
#pragma unroll
            for (int i = 0; i < WF; ++i) {
                const uint16_t* rrow = nullptr;
                if constexpr (RES) {
                    const int ml = (wave * WF + i) * 32 + (lane & 31);
                    rrow = p.res + ((static_cast<int64_t>(img) * H + h0) * W + (ml < npix ? ml : 0)) * p.Cout + c0 +
                           4 * half;
                }
                uint2 rv[2][4];
                if constexpr (RES) {   // all eight residual loads first, one wait
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) rv[j][g] = *reinterpret_cast<const uint2*>(rrow + 32 * j + 8 * g);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * g + e];
                        if constexpr (RES) {
                            const uint2 t = rv[j][g];
                            v[0] += __uint_as_float(t.x << 16);
                            v[1] += __uint_as_float(t.x & 0xFFFF0000u);
                            v[2] += __uint_as_float(t.y << 16);
                            v[3] += __uint_as_float(t.y & 0xFFFF0000u);
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
                        *reinterpret_cast<uint2*>(hb + (sbase[i] ^ ((4 * j + g) << 4))) = make_uint2(lo, hi);
                    }
            }
        };
        if (p.res) {
            stage(std::true_type{});
        } else {
            stage(std::false_type{});
        }
        barrier();   // X_k+1: staging complete
    }
}

template <int WF>
hipError_t launch_res(const HaloArgs& a, const HaloPlan& pl, int act, hipStream_t s) {
    switch (act) {
        case kActNone:
            hipLaunchKernelGGL((conv_halo_res_kernel<WF, kActNone>), dim3(kRBlocks), dim3(512), 0, s, a, pl.th,
                               pl.row_tiles, pl.per_xcd);
            break;
        case kActRelu:
            hipLaunchKernelGGL((conv_halo_res_kernel<WF, kActRelu>), dim3(kRBlocks), dim3(512), 0, s, a, pl.th,
                               pl.row_tiles, pl.per_xcd);
            break;
        case kActGelu:
            hipLaunchKernelGGL((conv_halo_res_kernel<WF, kActGelu>), dim3(kRBlocks), dim3(512), 0, s, a, pl.th,
                               pl.row_tiles, pl.per_xcd);
            break;
        case kActGeluErf:
            hipLaunchKernelGGL((conv_halo_res_kernel<WF, kActGeluErf>), dim3(kRBlocks), dim3(512), 0, s, a, pl.th,
                               pl.row_tiles, pl.per_xcd);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- small images (halo of a 64-channel group <= 32 KB): one image per workgroup ----
//
// For late-stage layers (e.g. 14 x 14 x 256) a row tile is too small to amortise the
// weights: a 64-channel output tile streams all 9 Cin x 64 weights for ~100 pixels.  Here a
// workgroup takes a whole image and 32 output channels, halving the weight bytes per CU, and
// streams the input halo by 64-channel groups through three 32 KB buffers in the order the
// contraction uses them: k runs channel group by channel group, and within a group over the
// nine taps, so groups q + 1 and q + 2 load while the taps of group q run.  Weight slices
// (32 rows x one tap x 64 channels, 4 KB) stream through a twelve-stage ring.
//
// This tiling reads 1.5 KB of fragments from LDS per MFMA, and a wave can keep at most 15
// LDS reads in flight, so eight waves issue them: waves w and w + 4 own the same 64 pixels x
// 32 channels and split every 32-channel k-step into its two 16-channel halves; the second
// wave's partial sums join the first's through LDS at the end.  Fragments are read two slices
// (four k-steps) ahead, and the slice barriers leave those reads in flight.  The loads into
// LDS use the buffer form: with the global (FLAT) form in flight the compiler cannot count
// outstanding LDS reads and waits for all of them before MFMAs.
constexpr int kIGroup = 32 * 1024;       // one halo channel group: (H+2)(W+2) pixels x 128 B
constexpr int kIG = 3;                   // halo group buffers
constexpr int kIS = 12;                  // weight ring stages (11 slices of lookahead)
constexpr int kILook = 2;                // fragments are read kILook slices (2 kILook steps) ahead
constexpr int kIB = 6;                   // fragment register buffers (> 2 kILook, divides 18)
constexpr int kISlice = 32 * 128;        // 32 output channels x 64 input channels x 2 B
constexpr int kIGLoads = kIGroup / 8192; // halo group pieces per wave (1 KB each, 8 waves)
// LDS reads a wave may leave in flight at a slice barrier: the reads of the last 2 kILook
// steps (three per step).  The buffers refilled after the barrier of slice kt were last read
// for slice kt - 1, whose reads went out 2 kILook steps before that slice, so they are older.
constexpr int kIKeep = 2 * kILook * 3;

template <int ACT>
__global__ __launch_bounds__(512, 1) void conv_halo_img_kernel(const HaloArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kIG * kIGroup + kIS * kISlice];
    uint8_t* const ring = smem + kIG * kIGroup;
    const int tid = static_cast<int>(threadIdx.x);
    // the wave index is uniform: in a scalar register the role branches below stay scalar
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), half = lane >> 5;
    const int pg = wave & 3, kh = wave >> 2;   // pixel fragments 2 pg, 2 pg + 1; k half
    const int bid = static_cast<int>(blockIdx.x);
    const int img = bid % p.N, ct = bid / p.N;   // the output tiles of one image share an XCD when N % 8 == 0
    const int c0 = ct * 32;
    const int H = p.H, W = p.W, W2 = p.W + 2, Cin = p.Cin;
    const int HW = H * W, NQ = (H + 2) * W2;
    const int Q = Cin >> 6, KT = 9 * Q, K = 9 * Cin;
    // this image's input and this tile's 32 weight rows as buffers (both well below 4 GB:
    // H W <= 256 pixels); loads outside the image or past the last slice read zeros
    const __amdgpu_buffer_rsrc_t xr =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.x) + static_cast<int64_t>(img) * HW * Cin * 2,
                    static_cast<uint32_t>(HW * Cin * 2));
    const __amdgpu_buffer_rsrc_t wr_ =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(p.w) + static_cast<int64_t>(c0) * K * 2,
                    static_cast<uint32_t>(32 * K * 2));

    // halo group q (channels 64 q .. 64 q + 63) into buffer q % kIG: pixel-major, 128 B per pixel,
    // chunk position c holds chunk c ^ hswz(pixel); kIGLoads pieces of 1 KB per wave
    auto load_group = [&](int q) {
        uint8_t* const buf = smem + (q % kIG) * kIGroup;
        const int nhi = (NQ * 128 + 1023) >> 10;
#pragma unroll
        for (int n = 0; n < kIGLoads; ++n) {
            const int li = wave + 8 * n;
            const int qq = li * 8 + (lane >> 3), pc = lane & 7;
            const int hr = qq / W2, wc = qq - hr * W2;
            const int hi = hr - 1, wi = wc - 1;
            const bool ok = li < nhi && qq < NQ && static_cast<unsigned>(hi) < static_cast<unsigned>(H) &&
                            static_cast<unsigned>(wi) < static_cast<unsigned>(W);
            const uint32_t off = static_cast<uint32_t>(((hi * W + wi) * Cin + q * 64 + ((pc ^ hswz(hr, wc, W)) << 3)) * 2);
            load_lds16_buf(xr, ok ? off : kOutOfRange, buf + li * 1024);
        }
    };
    // weight slice kt = (group kt / 9, tap kt % 9): rows c0 .. c0+31, 64 channels; waves 0-3 load
    // 8 rows each; past KT the zero page keeps their load count uniform
    const int wr = (wave & 3) * 8 + (lane >> 3);
    const uint32_t wrow = static_cast<uint32_t>((wr * K + wchunk(wr, lane & 7) * 8) * 2);
    auto issue_w = [&](int kt) {
        uint8_t* const st = ring + (kt % kIS) * kISlice + (wave & 3) * 1024;
        const int q = kt / 9, t = kt - q * 9;
        load_lds16_buf(wr_, kt < KT ? wrow + static_cast<uint32_t>((t * Cin + q * 64) * 2) : kOutOfRange, st);
    };

    // this wave's pixels: fragment i holds image pixel (2 pg + i) * 32 + lane % 32; the halo
    // address of each tap's pixel with swizzle and half folded in (chunk 2 u + half of 16-channel
    // sub-step u is at xa ^ (32 u))
    int xa[2][9];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pix = (2 * pg + i) * 32 + (lane & 31);
        const int pp = pix < HW ? pix : 0;
        const int ho = pp / W, wo = pp - ho * W;
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const int hr = ho + t / 3, wc = wo + t % 3;
            xa[i][t] = ((hr * W2 + wc) * 128 + (hswz(hr, wc, W) << 4)) ^ (half << 4);
        }
    }
    // this wave's sub-step of k-step s is u = 2 s + kh; weight row lane % 32, chunk 2 u + half
    const int row = lane & 31;
    int wo2[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) wo2[s2] = row * 128 + (((2 * (2 * s2 + kh) + half) ^ ((row >> 1) & 7)) << 4);
    f32x16_t biasv;   // the bias enters the first MFMA of the k-half-0 waves only
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        f32x4_t b4 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (p.bias && kh == 0) b4 = *reinterpret_cast<const f32x4_t*>(p.bias + c0 + 8 * g + 4 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) biasv[4 * g + e] = b4[e];
    }

    // the residual of this wave's outputs, loaded before anything else: the oldest loads, they
    // are complete by the prologue's wait for the first slices (loads return in issue order), so
    // none of the waits below counts them, and their latency hides behind the halo's
    uint2 rv[2][4];
    if (kh == 0 && p.res) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pix = (2 * pg + i) * 32 + (lane & 31);
            const int64_t e0 = (static_cast<int64_t>(img) * HW + (pix < HW ? pix : 0)) * p.Cout + c0 + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g) rv[i][g] = *reinterpret_cast<const uint2*>(p.res + e0 + 8 * g);
        }
    }

    // ---- prologue: groups 0 and 1, weight slices 0 .. kIS-2; slices 0 .. kILook visible ----
    load_group(0);
    if (Q > 1) load_group(1);
    if (kh == 0) {
#pragma unroll
        for (int kt = 0; kt < kIS - 1; ++kt) issue_w(kt);
        wait_vmcnt<kIS - 2 - kILook>();
    } else {
        if (Q > 1) {
            wait_vmcnt<kIGLoads>();   // group 0
        } else {
            wait_vmcnt<0>();
        }
    }
    barrier();

    f32x16_t acc[2];
    bf16x8_t xf[kIB][2], wf[kIB];   // buffer = step % kIB
    // fragments of global step gs (slice gs / 2, this wave's 16 channels of its 32-channel
    // step gs % 2); steps past the end re-read the last one (values unused)
    auto rd = [&](auto b_c, int gs) {
        constexpr int b = decltype(b_c)::value;
        gs = gs < 2 * KT ? gs : 2 * KT - 1;
        const int kt = gs >> 1, s2 = gs & 1;
        const int q = kt / 9, t = kt - q * 9;
        const uint8_t* const hb = smem + (q % kIG) * kIGroup;
        const int u = 2 * s2 + kh;
#pragma unroll
        for (int i = 0; i < 2; ++i) xf[b][i] = *reinterpret_cast<const bf16x8_t*>(hb + (xa[i][t] ^ (32 * u)));
        wf[b] = *reinterpret_cast<const bf16x8_t*>(ring + (kt % kIS) * kISlice + wo2[s2]);
    };
    auto mma = [&](auto b_c, bool first) {
        constexpr int b = decltype(b_c)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b], xf[b][i], first ? biasv : acc[i], 0, 0, 0);
    };
    static_for<0, 2 * kILook>([&](auto g_c) { rd(g_c, decltype(g_c)::value); });
    // Step gs reads step gs + 2 kILook, i.e. slice kt + kILook during slice kt, so that slice must
    // be visible when slice kt starts.  One iteration is a channel group: 9 slices = 18 steps,
    // a multiple of kIB, so every register buffer index is a compile-time constant.
    for (int q = 0; q < Q; ++q) {
        static_for<0, 18>([&](auto r_c) {
            constexpr int r = decltype(r_c)::value;
            const int kt = 9 * q + r / 2;
            if constexpr (r % 2 == 0) {
                if (kt > 0) {
                    if (kh == 0) {
                        // loads issued after slice kt + kILook's: slices kt + kILook + 1 ..
                        // kt + kIS - 2 and the halo groups issued at slices in
                        // [kt + kILook + 1 - kIS, kt - 1]: group m + 2 goes out at slice 9 m, so
                        // a window of kIS - kILook - 1 <= 18 slices holds at most two
                        static_assert(kIS - kILook - 1 <= 18, "at most two group loads per window");
                        const int lo = max(0, kt + kILook + 1 - kIS);
                        const int ng = max(0, min((kt - 1) / 9, Q - 3) - (lo + 8) / 9 + 1);
                        if (ng >= 2) {
                            wait_vm_lgkm<kIS - 2 - kILook + 2 * kIGLoads, kIKeep>();
                        } else if (ng == 1) {
                            wait_vm_lgkm<kIS - 2 - kILook + kIGLoads, kIKeep>();
                        } else {
                            wait_vm_lgkm<kIS - 2 - kILook, kIKeep>();
                        }
                    } else {
                        // this wave loads halo groups only: the group slice kt + kILook reads
                        // (clamped to the last) and the newer ones issued since
                        const int need = min(kt + kILook, KT - 1) / 9;
                        const int newest = min(Q - 1, max(Q > 1 ? 1 : 0, (kt - 1) / 9 + 2));
                        const int after = newest - need;
                        if (after <= 0) {
                            wait_vm_lgkm<0, kIKeep>();
                        } else if (after == 1) {
                            wait_vm_lgkm<kIGLoads, kIKeep>();
                        } else {
                            wait_vm_lgkm<2 * kIGLoads, kIKeep>();
                        }
                    }
                    barrier();
                }
                if (kh == 0) issue_w(kt + kIS - 1);
                if (r == 0 && q + 2 < Q) load_group(q + 2);
            }
            const int gs = 18 * q + r;
            rd(std::integral_constant<int, (r + 2 * kILook) % kIB>{}, gs + 2 * kILook);
            mma(std::integral_constant<int, r % kIB>{}, q == 0 && r == 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    wait_vmcnt<0>();

    // ---- the two k halves meet: waves 4-7 hand their partial sums to waves 0-3 through LDS ----
    barrier();   // every wave is done with the halo buffers
    float* const red = reinterpret_cast<float*>(smem) + pg * 2 * 16 * 64 + lane;
    if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[(i * 16 + e) * 64] = acc[i][e];
    }
    barrier();
    if (kh == 1) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] += red[(i * 16 + e) * 64];

    // ---- epilogue (bias already in acc): residual, activation, 8-byte stores of channels
    //      c0 + 8 g + 4 half .. +3 ----
    uint8_t* const yb = reinterpret_cast<uint8_t*>(p.y);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pix = (2 * pg + i) * 32 + (lane & 31);
        if (pix >= HW) continue;
        const int64_t e0 = (static_cast<int64_t>(img) * HW + pix) * p.Cout + c0 + 4 * half;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][4 * g + e];
            if (p.res) {
                v[0] += __uint_as_float(rv[i][g].x << 16);
                v[1] += __uint_as_float(rv[i][g].x & 0xFFFF0000u);
                v[2] += __uint_as_float(rv[i][g].y << 16);
                v[3] += __uint_as_float(rv[i][g].y & 0xFFFF0000u);
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
            *reinterpret_cast<uint2*>(yb + (e0 + 8 * g) * 2) = make_uint2(lo, hi);
        }
    }
}

hipError_t launch_img(const HaloArgs& a, int act, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.N * (a.Cout / 32))), block(512);
    switch (act) {
        case kActNone: hipLaunchKernelGGL((conv_halo_img_kernel<kActNone>), grid, block, 0, s, a); break;
        case kActRelu: hipLaunchKernelGGL((conv_halo_img_kernel<kActRelu>), grid, block, 0, s, a); break;
        case kActGelu: hipLaunchKernelGGL((conv_halo_img_kernel<kActGelu>), grid, block, 0, s, a); break;
        case kActGeluErf: hipLaunchKernelGGL((conv_halo_img_kernel<kActGeluErf>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int WF, int HALO_KB>
hipError_t launch_act(const HaloArgs& a, int th, int row_tiles, int act, hipStream_t s) {
    const int blocks = a.N * row_tiles * a.co_tiles;
    switch (act) {
        case kActNone:
            hipLaunchKernelGGL((conv_halo_kernel<WF, HALO_KB, kActNone>), dim3(blocks), dim3(256), 0, s, a, th, row_tiles);
            break;
        case kActRelu:
            hipLaunchKernelGGL((conv_halo_kernel<WF, HALO_KB, kActRelu>), dim3(blocks), dim3(256), 0, s, a, th, row_tiles);
            break;
        case kActGeluErf:
            hipLaunchKernelGGL((conv_halo_kernel<WF, HALO_KB, kActGeluErf>), dim3(blocks), dim3(256), 0, s, a, th, row_tiles);
            break;
        case kActGelu:
            hipLaunchKernelGGL((conv_halo_kernel<WF, HALO_KB, kActGelu>), dim3(blocks), dim3(256), 0, s, a, th, row_tiles);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Tile plan for the halo kernel, or false when the shape does not qualify.
bool conv_halo_plan(int N, int H, int W, int Cin, int Cout, bool resident_ok, HaloPlan* plan) {
    if (N <= 0 || H <= 0 || W <= 0 || Cout <= 0 || Cout % kCo != 0) return false;
    // Cin = 64: resident weights when 32 workgroups per XCD divide evenly among the output
    // tiles and a halo of at least one row fits its 44 KB buffer
    const int co_tiles = Cout / kCo;
    if (resident_ok && Cin == 64 && 32 % co_tiles == 0 && W <= 256 && 3 * (W + 2) * 128 <= kRHalo &&
        static_cast<int64_t>(H) * W * 128 < (int64_t(1) << 31)) {
        int th = 256 / W;
        if (th > H) th = H;
        while (th > 1 && (th + 2) * (W + 2) * 128 > kRHalo) --th;
        const int64_t tiles = static_cast<int64_t>(N) * ((H + th - 1) / th);
        if (tiles <= 0x7fffffff) {
            plan->kind = 1;
            plan->th = th;
            plan->row_tiles = (H + th - 1) / th;
            plan->wf = th * W <= 128 ? 1 : 2;
            plan->halo_kb = 44;
            plan->per_xcd = static_cast<int>((tiles + 7) / 8);
            return true;
        }
    }
    // small images: the whole image per workgroup (kind 2) when that still gives >= 128 workgroups
    if (resident_ok && Cin % 64 == 0 && Cin > 0 && Cout % 32 == 0 && H * W <= 256 && (H + 2) * (W + 2) * 128 <= kIGroup &&
        static_cast<int64_t>(N) * (Cout / 32) >= 128 && static_cast<int64_t>(N) * (Cout / 32) <= 0x7fffffff) {
        plan->kind = 2;
        plan->th = H;
        plan->row_tiles = 1;
        plan->wf = 2;
        plan->halo_kb = kIG * kIGroup / 1024;
        plan->per_xcd = 0;
        return true;
    }
    if (Cin != 64 && (Cin <= 0 || Cin % 128 != 0)) return false;   // the halo swizzle stays inside a pixel
    if (Cin > 1024 || W > 256) return false;
    if (static_cast<int64_t>(H) * W * Cin * 2 >= (int64_t(1) << 31)) return false;   // 32-bit buffer offsets
    const int ps = Cin * 2;
    int th = 256 / W;                      // at most 8 fragments of 32 pixels
    if (th > H) th = H;
    if (th < 1) return false;
    auto halo_kb = [&](int t) { return (((t + 2) * (W + 2) * ps) + 1023) / 1024; };
    while (th > 1 && halo_kb(th) > 96) --th;
    if (halo_kb(th) > 96) return false;
    // equal row tiles: the fewest tiles at this height, then the smallest height giving that many
    auto balance = [&](int t) { const int rt = (H + t - 1) / t; return (H + rt - 1) / rt; };
    th = balance(th);
    // enough workgroups to occupy the chip
    auto blocks = [&](int t) { return static_cast<int64_t>(N) * ((H + t - 1) / t) * (Cout / kCo); };
    while (th > 1 && blocks(th) < 256) th = balance((th + 1) / 2);
    if (static_cast<int64_t>(N) * ((H + th - 1) / th) * (Cout / kCo) > 0x7fffffff) return false;
    const int frags = (th * W + 31) / 32;
    plan->kind = 0;
    plan->per_xcd = 0;
    plan->th = th;
    plan->row_tiles = (H + th - 1) / th;
    plan->wf = frags <= 4 ? 1 : 2;
    plan->halo_kb = halo_kb(th) <= 48 ? 48 : 96;
    return true;
}

hipError_t launch_conv_halo(const HaloArgs& a, const HaloPlan& plan, int act, hipStream_t s) {
    if (plan.kind == 2) return launch_img(a, act, s);
    if (plan.kind == 1) return plan.wf == 1 ? launch_res<1>(a, plan, act, s) : launch_res<2>(a, plan, act, s);
    if (plan.wf == 1)
        return plan.halo_kb == 48 ? launch_act<1, 48>(a, plan.th, plan.row_tiles, act, s)
                                  : launch_act<1, 96>(a, plan.th, plan.row_tiles, act, s);
    return plan.halo_kb == 48 ? launch_act<2, 48>(a, plan.th, plan.row_tiles, act, s)
                              : launch_act<2, 96>(a, plan.th, plan.row_tiles, act, s);
}

}  // namespace dlf
