// MFMA GEMM / implicit-GEMM kernel for gfx950 with a register epilogue.
//
// One workgroup (4 waves, 256 lanes) owns a BM x BN tile of C.  The K loop
// stages 128-byte-wide slices of A and B (64 bf16 or 128 fp8 per row) through
// LDS with a double buffer: while the MFMAs consume slice k, the next slice is
// already in flight from global memory into registers and is written to the
// other LDS buffer afterwards (one barrier per slice).  LDS rows are XOR-
// swizzled in 16-byte chunks so that both the row-wise stores and the MFMA
// fragment reads (32 rows x one chunk) are bank-conflict free.
//
// The contraction uses v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x64_f8f6f4
// (fp8 e4m3 x e4m3) with fp32 accumulators that stay in registers; the
// epilogue then applies per-column scale/shift (folded BN or bias), the
// residual and the activation to those registers and stores each output
// element once.  That is the conv implicit-GEMM main loop plus epilogue of
// "OpenPPL算子融合深度解析" §4.3, with the FP8 static-scale store of
// "FlashRT 跨层融合深度解析" §3.
//
// For a convolution the A operand is never materialised: row m = (img, ho, wo)
// and column k = (r*KW + s)*Cin + ci are gathered from the NHWC input while
// loading, with zero fill outside the image (zero padding as in the direct
// convolution loop of the discosf.com fusion article §3.3).
#include "device_common.h"
#include "kernels.h"

namespace dlf {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // one LDS row of a K slice

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 MFMA fragments per wave
    static constexpr int AR = BM / 32, BR = BN / 32;     // rows each lane loads per slice
    static constexpr int STAGE = (BM + BN) * kRowBytes;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32x32 fragments");
};

// Byte offset of 16-byte chunk `chunk` of LDS row `row` (XOR swizzle over 8 chunks).
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Maps the linear workgroup id to an output tile.  Consecutive workgroup ids are
// dealt round-robin to the 8 XCDs (each with its own L2), so ids are first
// regrouped so that each XCD receives a contiguous range of tiles; within the
// range, tiles are ordered in groups of 8 tile-rows that sweep all tile-columns,
// so the tiles resident on one XCD at a time share A rows and B columns in L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nb = tiles_m * tiles_n;
    const int bid = static_cast<int>(blockIdx.x);
    const int xcd = bid & 7, local = bid >> 3;
    const int q = nb >> 3, r = nb & 7;
    const int id = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    constexpr int G = 8;
    const int per_group = G * tiles_n;
    const int g = id / per_group;
    const int first_m = g * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in_g = id - g * per_group;
    tm = first_m + in_g % gsize;
    tn = in_g / gsize;
}

template <int ELEM>
struct Frag;

template <>
struct Frag<2> {   // bf16: 16-wide K per MFMA, 8 elements (one chunk) per lane
    using T = bf16x8_t;
    static constexpr int kSlices = 4;   // 64 K per 128-byte row
    static __device__ __forceinline__ T load(const uint8_t* s, int row, int kk, int lane) {
        return *reinterpret_cast<const T*>(s + swz(row, kk * 2 + (lane >> 5)));
    }
    static __device__ __forceinline__ f32x16_t mma(const T& a, const T& b, const f32x16_t& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Frag<1> {   // fp8 e4m3: 64-wide K per MFMA, 32 elements (two chunks) per lane
    using T = i32x8_t;
    static constexpr int kSlices = 2;   // 128 K per 128-byte row
    static __device__ __forceinline__ T load(const uint8_t* s, int row, int kk, int lane) {
        const int c0 = kk * 4 + (lane >> 5) * 2;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(s + swz(row, c0));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(s + swz(row, c0 + 1));
        T r;
        r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
        r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
        return r;
    }
    static __device__ __forceinline__ f32x16_t mma(const T& a, const T& b, const f32x16_t& c) {
        // format 0 = e4m3 for both operands; zero scale operands select the unscaled MFMA
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

template <int ELEM, class TS, bool CONV, int ACT, int OUT>
__global__ __launch_bounds__(kThreads, 1) void mma_kernel(const MmaArgs p, const int tiles_m,
                                                          const int tiles_n) {
    constexpr int CE = 16 / ELEM;            // elements per 16-byte chunk
    constexpr int KE = kRowBytes / ELEM;     // K elements per slice
    using F = Frag<ELEM>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TS::STAGE];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / TS::WAVES_N, wn = wave % TS::WAVES_N;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * TS::BM;
    const int n0 = tn * TS::BN;
    const int64_t M = p.M;
    const int N = p.N, K = p.K;

    // ---- loader state: this lane moves chunk lc of rows lr + 32 i ----
    const int lc = tid & 7, lr = tid >> 3;
    const uint8_t* const a_bytes = static_cast<const uint8_t*>(p.a);
    const uint8_t* const b_bytes = static_cast<const uint8_t*>(p.b);
    const int64_t row_bytes = static_cast<int64_t>(K) * ELEM;

    uint32_t a_ok = 0, b_ok = 0;          // per-row validity bits
    int a_pix[CONV ? TS::AR : 1], a_h[CONV ? TS::AR : 1], a_w[CONV ? TS::AR : 1];
#pragma unroll
    for (int i = 0; i < TS::AR; ++i) {
        const int64_t m = m0 + lr + 32 * i;
        if (m < M) a_ok |= 1u << i;
        if constexpr (CONV) {
            const int mm = static_cast<int>(m < M ? m : 0);
            const int hw = p.Ho * p.Wo;
            const int img = mm / hw, rem = mm - img * hw;
            const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
            a_h[i] = ho * p.SH - p.PH;
            a_w[i] = wo * p.SW - p.PW;
            a_pix[i] = (img * p.H + a_h[i]) * p.W + a_w[i];
        }
    }
#pragma unroll
    for (int i = 0; i < TS::BR; ++i)
        if (n0 + lr + 32 * i < N) b_ok |= 1u << i;

    const uint8_t* const a_row0 = a_bytes + (m0 + lr) * row_bytes + lc * 16;
    const uint8_t* const b_row0 = b_bytes + static_cast<int64_t>(n0 + lr) * row_bytes + lc * 16;

    u32x4_t ra[TS::AR], rb[TS::BR];
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    auto global_load = [&](int kt) {
        const int kb = kt * KE + lc * CE;     // first K element of this lane's chunk
        const bool kin = kb < K;
        if constexpr (CONV) {
            int r = 0, s = 0, ci = 0;
            if (kin) {
                const int tap = kb / p.Cin;
                ci = kb - tap * p.Cin;
                r = tap / p.KW;
                s = tap - r * p.KW;
            }
#pragma unroll
            for (int i = 0; i < TS::AR; ++i) {
                const int hi = a_h[i] + r, wi = a_w[i] + s;
                const bool ok = kin && ((a_ok >> i) & 1u) && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                                static_cast<unsigned>(wi) < static_cast<unsigned>(p.W);
                const int64_t off = (static_cast<int64_t>(a_pix[i] + r * p.W + s) * p.Cin + ci) * ELEM;
                ra[i] = ok ? *reinterpret_cast<const u32x4_t*>(a_bytes + off) : zero;
            }
        } else {
#pragma unroll
            for (int i = 0; i < TS::AR; ++i) {
                const bool ok = kin && ((a_ok >> i) & 1u);
                ra[i] = ok ? *reinterpret_cast<const u32x4_t*>(a_row0 + 32 * i * row_bytes + kt * kRowBytes)
                           : zero;
            }
        }
#pragma unroll
        for (int i = 0; i < TS::BR; ++i) {
            const bool ok = kin && ((b_ok >> i) & 1u);
            rb[i] = ok ? *reinterpret_cast<const u32x4_t*>(b_row0 + 32 * i * row_bytes + kt * kRowBytes)
                       : zero;
        }
    };
    auto lds_store = [&](int stage) {
        uint8_t* sA = smem + stage * TS::STAGE;
        uint8_t* sB = sA + TS::BM * kRowBytes;
#pragma unroll
        for (int i = 0; i < TS::AR; ++i)
            *reinterpret_cast<u32x4_t*>(sA + swz(lr + 32 * i, lc)) = ra[i];
#pragma unroll
        for (int i = 0; i < TS::BR; ++i)
            *reinterpret_cast<u32x4_t*>(sB + swz(lr + 32 * i, lc)) = rb[i];
    };

    f32x16_t acc[TS::FM][TS::FN];
#pragma unroll
    for (int i = 0; i < TS::FM; ++i)
#pragma unroll
        for (int j = 0; j < TS::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int KT = (K + KE - 1) / KE;
    if (KT > 0) {
        global_load(0);
        lds_store(0);
    }
    __syncthreads();

    const int a_frag_row = wm * TS::WTM + (lane & 31);
    const int b_frag_row = wn * TS::WTN + (lane & 31);
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) global_load(kt + 1);
        const uint8_t* sA = smem + cur * TS::STAGE;
        const uint8_t* sB = sA + TS::BM * kRowBytes;
#pragma unroll
        for (int kk = 0; kk < F::kSlices; ++kk) {
            typename F::T af[TS::FM], bfr[TS::FN];
#pragma unroll
            for (int i = 0; i < TS::FM; ++i) af[i] = F::load(sA, a_frag_row + 32 * i, kk, lane);
#pragma unroll
            for (int j = 0; j < TS::FN; ++j) bfr[j] = F::load(sB, b_frag_row + 32 * j, kk, lane);
#pragma unroll
            for (int i = 0; i < TS::FM; ++i)
#pragma unroll
                for (int j = 0; j < TS::FN; ++j) acc[i][j] = F::mma(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < KT) lds_store(cur ^ 1);
        __syncthreads();
    }

    // ---- register epilogue: lane holds column (lane & 31) and 16 rows per fragment:
    //      row = 8*(e/4) + 4*(lane/32) + e%4 within the 32x32 fragment ----
    const float* const scale = p.scale;
    const float* const shift = p.shift;
#pragma unroll
    for (int j = 0; j < TS::FN; ++j) {
        const int col = n0 + wn * TS::WTN + 32 * j + (lane & 31);
        const bool col_ok = col < N;
        float sc = 1.0f, sh = 0.0f;
        if (col_ok) {
            if (scale) sc = scale[col];
            if (shift) sh = shift[col];
        }
#pragma unroll
        for (int i = 0; i < TS::FM; ++i) {
            const int64_t rbase = m0 + wm * TS::WTM + 32 * i + 4 * (lane >> 5);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = rbase + 8 * (e >> 2) + (e & 3);
                if (!col_ok || row >= M) continue;
                const int64_t idx = row * N + col;
                float v = acc[i][j][e];
                if constexpr (OUT == kOutF32) {
                    static_cast<float*>(p.c)[idx] = v * p.dequant;
                } else {
                    v = scale ? fmaf(v, sc, sh) : v + sh;
                    if (p.res) v += bf16_to_f32(p.res[idx]);
                    v = activate<ACT>(v);
                    if constexpr (OUT == kOutFp8)
                        static_cast<uint8_t*>(p.c)[idx] = static_cast<uint8_t>(quant_e4m3(v, p.out_inv_scale));
                    else
                        static_cast<uint16_t*>(p.c)[idx] = f32_to_bf16(v);
                }
            }
        }
    }
}

using T256x256 = TileShape<256, 256, 2, 2>;
using T128x128 = TileShape<128, 128, 2, 2>;
using T256x64 = TileShape<256, 64, 4, 1>;
using T64x64 = TileShape<64, 64, 2, 2>;
using T128x64 = TileShape<128, 64, 2, 2>;

template <int ELEM, class TS, bool CONV, int ACT, int OUT>
hipError_t launch_one(const MmaArgs& a, hipStream_t stream) {
    const int64_t tm64 = (a.M + TS::BM - 1) / TS::BM;
    const int tiles_n = (a.N + TS::BN - 1) / TS::BN;
    if (tm64 * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>(tm64);
    if (tiles_m == 0 || tiles_n == 0) return hipSuccess;
    hipLaunchKernelGGL((mma_kernel<ELEM, TS, CONV, ACT, OUT>), dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                       stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int ELEM, bool CONV, int ACT, int OUT>
hipError_t launch_tile(const MmaArgs& a, int tile, hipStream_t s) {
    switch (tile) {
        case kTile256x256: return launch_one<ELEM, T256x256, CONV, ACT, OUT>(a, s);
        case kTile128x128: return launch_one<ELEM, T128x128, CONV, ACT, OUT>(a, s);
        case kTile256x64: return launch_one<ELEM, T256x64, CONV, ACT, OUT>(a, s);
        case kTile64x64: return launch_one<ELEM, T64x64, CONV, ACT, OUT>(a, s);
        case kTile128x64: return launch_one<ELEM, T128x64, CONV, ACT, OUT>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int mma_tile_rows(int tile) {
    switch (tile) {
        case kTile256x256: case kTile256x64: return 256;
        case kTile128x128: case kTile128x64: return 128;
        case kTile64x64: return 64;
        default: return 0;
    }
}

int mma_tile_cols(int tile) {
    switch (tile) {
        case kTile256x256: return 256;
        case kTile128x128: return 128;
        default: return 64;
    }
}

hipError_t launch_mma_bf16(const MmaArgs& a, bool conv, int act, int tile, hipStream_t s) {
    if (conv) {
        switch (act) {
            case kActNone: return launch_tile<2, true, kActNone, kOutBf16>(a, tile, s);
            case kActRelu: return launch_tile<2, true, kActRelu, kOutBf16>(a, tile, s);
            case kActGelu: return launch_tile<2, true, kActGelu, kOutBf16>(a, tile, s);
        }
    } else {
        switch (act) {
            case kActNone: return launch_tile<2, false, kActNone, kOutBf16>(a, tile, s);
            case kActRelu: return launch_tile<2, false, kActRelu, kOutBf16>(a, tile, s);
            case kActGelu: return launch_tile<2, false, kActGelu, kOutBf16>(a, tile, s);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mma_fp8(const MmaArgs& a, int act, int out, int tile, hipStream_t s) {
    if (out == kOutF32) return act == kActNone ? launch_tile<1, false, kActNone, kOutF32>(a, tile, s)
                                               : hipErrorInvalidValue;
    if (out == kOutFp8) {
        if (act == kActNone) return launch_tile<1, false, kActNone, kOutFp8>(a, tile, s);
        if (act == kActRelu) return launch_tile<1, false, kActRelu, kOutFp8>(a, tile, s);
    }
    if (out == kOutBf16) {
        if (act == kActNone) return launch_tile<1, false, kActNone, kOutBf16>(a, tile, s);
        if (act == kActRelu) return launch_tile<1, false, kActRelu, kOutBf16>(a, tile, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dlf
