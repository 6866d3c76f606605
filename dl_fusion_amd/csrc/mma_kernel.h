// MFMA GEMM / implicit-GEMM kernel for gfx950 with a register epilogue (the kernel template,
// its tile shapes and the tile switch; each mma_*.hip instantiates one group of it, so that the
// groups compile in parallel).
//
// One workgroup (4 or 16 waves) owns a BM x BN tile of C.  The K loop
// streams 64-byte slices of every A and B row (32 bf16 or 64 fp8 values)
// straight from global memory into a ring of STAGES LDS buffers with
// global_load_lds_dwordx4 (no register staging), so STAGES-1 slices are in
// flight while the MFMAs consume the current one.  Each load instruction fills
// one contiguous kilobyte of LDS (16 rows); the lane -> row/chunk assignment
// applies an XOR swizzle on the 16-byte chunks so that the MFMA operand reads
// (32 rows x one chunk per instruction) are free of bank conflicts.  Lanes
// whose chunk lies outside the operand (M/N/K tails, convolution padding) read
// a zero page instead, so the LDS image is exactly the zero-padded operand.
//
// The contraction is v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x64_f8f6f4
// (e4m3 x e4m3) with fp32 accumulators that stay in registers.  The MFMA is
// issued as D = W . X^T, so each lane holds one output row and runs of four
// consecutive output columns; the epilogue applies the per-column scale/shift
// (folded BN or bias), the residual and the activation on those registers,
// rounds once, and stages the tile through LDS so that every output element
// is written to global memory exactly once by a coalesced 16-byte store.  This
// is the conv implicit-GEMM main loop plus epilogue of
// "OpenPPL算子融合深度解析" §4.3, with the static-scale FP8 store of
// "FlashRT 跨层融合深度解析" §3.
//
// For a convolution the A operand is never materialised: row m = (img, ho, wo)
// and column k = (r*KW + s)*Cin + ci are gathered from the NHWC input by the
// load addresses, with the zero page standing in for taps outside the image
// (zero padding as in the direct convolution loop of the discosf.com fusion
// article §3.3).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "mma_common.h"

namespace dlf {
namespace {

constexpr int kRowBytes = 64;      // bytes of each operand row per K slice
constexpr int kChunks = 4;         // 16-byte chunks per row slice
constexpr int kRowsPerLoad = 16;   // one load instruction fills 1 KB = 16 rows

// Zero-initialised device memory read by lanes whose chunk is padding.
__device__ __attribute__((aligned(64))) uint8_t g_zero_page[64];

// Operand A modes: dense rows read through a buffer resource per tile panel (32-bit offsets,
// rows below 8 MB), dense rows read by 64-bit global addresses (longer rows), or gathered
// from an NHWC convolution input.
// A operand: dense rows (32-bit buffer offsets, or 64-bit addresses for rows of 8 MB or more),
// or gathered from an NHWC image: a 64-byte slice inside one kernel tap (Cin % 32 == 0), a
// 16-byte chunk inside one tap (Cin % 8 == 0), or value by value (any Cin).
enum : int { kDense = 0, kConvAligned = 1, kConvGeneric = 2, kDenseWide = 3, kConvAnyC = 4 };

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int SPB_ = 1>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
    static constexpr int SPB = SPB_;                       // K slices consumed per barrier
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 fragments per wave
    static constexpr int NW = WAVES_M * WAVES_N;           // waves per workgroup
    static constexpr int NT = 64 * NW;                     // lanes per workgroup
    static constexpr int LA = BM / kRowsPerLoad / NW;      // A loads per lane per slice
    static constexpr int LB = BN / kRowsPerLoad / NW;      // B loads per lane per slice
    static constexpr int STAGE = (BM + BN) * kRowBytes;
    static_assert(NW == 4 || NW == 16, "four or sixteen waves per workgroup (one or four per SIMD)");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "whole 32x32 fragments");
    static_assert(LA >= 1 && LB >= 1, "each wave loads at least one kilobyte per operand");
    static_assert(STAGES >= 2 * SPB, "the ring holds the slices being read and the ones landing");
};

// Physical 16-byte chunk of logical chunk c in row r.  Rows are 64 bytes (four
// chunks), so rows r, r+4, r+8, r+12 start in the same bank group; XOR-ing the
// chunk with bits 2..3 of the row spreads the 16 rows that one fragment read
// serves per cycle over 16 distinct 16-byte bank groups (measured on gfx950 with
// SQ_LDS_BANK_CONFLICT: zero conflict cycles for both MFMA k-steps).
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowBytes + (swz_chunk(r, c) << 4); }

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
struct Frag<2> {   // bf16: 16 K per MFMA; a lane supplies 8 values (one chunk)
    using T = bf16x8_t;
    static constexpr int kSteps = 2;   // MFMA k-steps per 64-byte slice
    static constexpr int kReads = 1;   // LDS reads per fragment
    static __device__ __forceinline__ T load(const uint8_t* s, int row, int step, int lane) {
        return *reinterpret_cast<const T*>(s + lds_off(row, step * 2 + (lane >> 5)));
    }
    static __device__ __forceinline__ f32x16_t mma(const T& a, const T& b, const f32x16_t& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Frag<1> {   // fp8 e4m3: 64 K per MFMA; a lane supplies 32 values (two chunks)
    using T = i32x8_t;
    static constexpr int kSteps = 1;
    static constexpr int kReads = 2;
    static __device__ __forceinline__ T load(const uint8_t* s, int row, int, int lane) {
        const int c0 = (lane >> 5) * 2;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(s + lds_off(row, c0));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(s + lds_off(row, c0 + 1));
        T r;
        r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
        r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
        return r;
    }
    static __device__ __forceinline__ f32x16_t mma(const T& a, const T& b, const f32x16_t& c) {
        // operand format 0 = e4m3 for both; zero scale operands select the unscaled MFMA
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// The register epilogue and the store of one output tile: acc[j][i] of wave (wm, wn) holds
// rows m0 + wm*WTM + 32 i + (lane & 31) and, in register group g = e/4, columns
// n0 + wn*WTN + 32 j + 8 g + 4 (lane/32) + e%4.  Every wave of the workgroup calls it after its
// last LDS read of operands: the LDS (smem) is then reused to stage the rounded tile.
template <class TS, int AMODE, int ACT, int OUT>
__device__ __forceinline__ void mma_epilogue(const MmaArgs& p, f32x16_t (&acc)[TS::FN][TS::FM], uint8_t* smem,
                                             const int wm, const int wn, const int lane, const int tid,
                                             const int64_t m0, const int n0) {
    const int64_t M = p.M;
    const int N = p.N;
    // ---- epilogue.  Lane holds output row  m = m0 + wm*WTM + 32 i + (lane & 31)  and, in
    //      register group g = e/4, columns  n = n0 + wn*WTN + 32 j + 8 g + 4 (lane/32) + e%4 ----
    const int lrow = lane & 31, half = lane >> 5;
    if constexpr (OUT == kOutF32) {
        // fp32 result of the plain fp8 GEMM: acc * dequant, stored directly (16 B per lane-group)
#pragma unroll
        for (int j = 0; j < TS::FN; ++j)
#pragma unroll
            for (int i = 0; i < TS::FM; ++i) {
                const int64_t m = m0 + wm * TS::WTM + 32 * i + lrow;
                if (m >= M) continue;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * TS::WTN + 32 * j + 8 * g + 4 * half;
                    float* dst = static_cast<float*>(p.c) + m * N + n;
                    if (n + 3 < N && (N & 3) == 0) {
                        f32x4_t v;
                        for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * g + e] * p.dequant;
                        *reinterpret_cast<f32x4_t*>(dst) = v;
                    } else {
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) dst[e] = acc[j][i][4 * g + e] * p.dequant;
                    }
                }
            }
        return;
    } else {
        constexpr int OB = OUT == kOutFp8 ? 1 : 2;            // output bytes per element
        // gated: columns (2j, 2j+1) are (gate j, up j) and give output column j
        constexpr bool GATED = ACT >= kActSiluMul;
        static_assert(!GATED || (OUT == kOutBf16 && AMODE != kConvAligned && AMODE != kConvGeneric &&
                                 AMODE != kConvAnyC),
                      "gated epilogue: dense bf16 output");
        constexpr int SROW = (GATED ? TS::BN / 2 : TS::BN) * OB;   // staging row bytes
        constexpr int CPR = SROW / 16;                        // 16-byte chunks per staged row
        // staged chunk cc of row r lives at chunk cc ^ (r & XM): the 16 rows written by one
        // store instruction land in distinct bank groups instead of one
        constexpr int XM = (CPR < 16 ? CPR : 16) - 1;
        __syncthreads();   // all waves are done reading operand slices: the LDS is reused for staging
        const float* const scale = p.scale;
        const float* const shift = p.shift;
        const int64_t m_last = M - 1;
        const int n_last4 = N >= 4 ? N - 4 : 0;
#pragma unroll
        for (int j = 0; j < TS::FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * TS::WTN + 32 * j + 8 * g + 4 * half;   // first of 4 columns
                const int n = n0 + nl;
                // per-column parameters; columns past N read a clamped (valid) address and
                // their results are never written out
                float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f}, sh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if ((N & 3) == 0) {   // n % 4 == 0: the run of four is entirely in or past N
                    const int nc = min(n, n_last4);
                    if (scale) {
                        const f32x4_t t = *reinterpret_cast<const f32x4_t*>(scale + nc);
                        sc[0] = t[0]; sc[1] = t[1]; sc[2] = t[2]; sc[3] = t[3];
                    }
                    if (shift) {
                        const f32x4_t t = *reinterpret_cast<const f32x4_t*>(shift + nc);
                        sh[0] = t[0]; sh[1] = t[1]; sh[2] = t[2]; sh[3] = t[3];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int nc = min(n + e, N - 1);
                        if (scale) sc[e] = scale[nc];
                        if (shift) sh[e] = shift[nc];
                    }
                }
#pragma unroll
                for (int i = 0; i < TS::FM; ++i) {
                    const int ml = wm * TS::WTM + 32 * i + lrow;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = acc[j][i][4 * g + e];
                        v[e] = scale ? fmaf(t, sc[e], sh[e]) : t + sh[e];
                    }
                    if (!GATED && p.res != nullptr) {
                        const int64_t mc = min(m0 + ml, m_last);
                        if ((N & 3) == 0) {   // 8-byte aligned run of four
                            const uint2 t = *reinterpret_cast<const uint2*>(p.res + mc * N + min(n, n_last4));
                            v[0] += __uint_as_float(t.x << 16);
                            v[1] += __uint_as_float(t.x & 0xFFFF0000u);
                            v[2] += __uint_as_float(t.y << 16);
                            v[3] += __uint_as_float(t.y & 0xFFFF0000u);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(p.res[mc * N + min(n + e, N - 1)]);
                        }
                    }
                    if constexpr (GATED) {
                        // output columns nl/2 and nl/2 + 1 (nl % 4 == 0): one 4-byte staging write
                        const int cb = (nl >> 1) * OB;
                        uint8_t* dst = smem + ml * SROW + ((((cb >> 4) ^ (ml & XM))) << 4) + (cb & 15);
                        *reinterpret_cast<uint32_t*>(dst) =
                            pack_bf16x2(gate_act<ACT>(v[0]) * v[1], gate_act<ACT>(v[2]) * v[3]);
                        continue;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = activate<ACT>(v[e]);
                    const int cb = nl * OB;                               // byte column in the row
                    uint8_t* dst = smem + ml * SROW + ((((cb >> 4) ^ (ml & XM))) << 4) + (cb & 15);
                    if constexpr (OUT == kOutFp8) {
                        *reinterpret_cast<uint32_t*>(dst) = quant_e4m3_x4(v[0], v[1], v[2], v[3], p.out_inv_scale);
                    } else {
                        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(v[0])) |
                                            (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
                        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(v[2])) |
                                            (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
                        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                    }
                }
            }
        }
        __syncthreads();
        // coalesced write-out: 16-byte chunks of the staged tile, row-major
        if (!GATED && p.parts > 1) {
            // split store: a chunk lies in one part (the part width is a whole number of chunks)
            const int pc = p.part_cols;
            for (int q = tid; q < TS::BM * CPR; q += TS::NT) {
                const int ml = q / CPR, cc = q - ml * CPR;
                const int64_t m = m0 + ml;
                const int n = n0 + cc * (16 / OB);
                if (m >= M || n >= N) continue;
                const int part = (n >= pc) + (n >= 2 * pc) + (n >= 3 * pc);
                uint8_t* const base = static_cast<uint8_t*>(part == 0 ? p.outs[0] : part == 1 ? p.outs[1]
                                                            : part == 2 ? p.outs[2] : p.outs[3]);
                *reinterpret_cast<u32x4_t*>(base + (m * pc + (n - part * pc)) * OB) =
                    *reinterpret_cast<const u32x4_t*>(smem + ml * SROW + ((cc ^ (ml & XM)) << 4));
            }
            return;
        }
        const int NO = GATED ? N / 2 : N;                     // output columns
        const int no0 = GATED ? n0 / 2 : n0;                  // first output column of the tile
        const bool vec_ok = ((static_cast<int64_t>(NO) * OB) & 15) == 0;
        uint8_t* const cbytes = static_cast<uint8_t*>(p.c);
        for (int q = tid; q < TS::BM * CPR; q += TS::NT) {
            const int ml = q / CPR, cc = q - ml * CPR;
            const int64_t m = m0 + ml;
            const int nl = cc * (16 / OB);
            const int n = no0 + nl;
            if (m >= M || n >= NO) continue;
            const uint8_t* src = smem + ml * SROW + ((cc ^ (ml & XM)) << 4);
            uint8_t* dst = cbytes + (m * NO + n) * OB;
            if (vec_ok && n + 16 / OB <= NO) {
                *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
            } else {
                const int cnt = min(16 / OB, NO - n) * OB;
                for (int b = 0; b < cnt; ++b) dst[b] = src[b];
            }
        }
    }
}

template <int ELEM, class TS, int AMODE, int ACT, int OUT>
__global__ __launch_bounds__(TS::NT, 1) void mma_kernel(const MmaArgs p, const int tiles_m,
                                                          const int tiles_n) {
    constexpr bool DENSE = AMODE == kDense || AMODE == kDenseWide;
    // dense operands as buffers: the LDS-DMA loads are then not FLAT instructions, which
    // keeps the compiler's count of outstanding LDS reads exact while they are in flight, and
    // the offsets are 32-bit
    constexpr bool BUF = AMODE == kDense;
    constexpr int CE = 16 / ELEM;                 // elements per 16-byte chunk
    constexpr int KE = kRowBytes / ELEM;          // K elements per slice
    constexpr int S = TS::STAGES;
    // vmcnt units per slice per lane.  The value-by-value gather completes inside the slice's
    // issue (its values pass through registers into LDS), so it leaves none outstanding.
    constexpr int LOADS = AMODE == kConvAnyC ? 0 : TS::LA + TS::LB;
    using F = Frag<ELEM>;
    // the LDS holds the operand ring during the K loop and the rounded output tile after it
    constexpr int STAGED = OUT == kOutF32 ? 0 : TS::BM * TS::BN * (OUT == kOutFp8 ? 1 : 2);
    constexpr int SMEM = S * TS::STAGE > STAGED ? S * TS::STAGE : STAGED;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / TS::WAVES_N, wn = wave % TS::WAVES_N;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * TS::BM;
    const int n0 = tn * TS::BN;
    const int64_t M = p.M;
    const int N = p.N, K = p.K;
    const int KT = (K + KE - 1) / KE;

    // ---- load assignment: wave w fills kilobytes [w*LA, (w+1)*LA) of the A slice and
    //      [w*LB, ...) of the B slice; lane i writes row 16*kb + i/4, physical chunk i%4 ----
    const uint8_t* const a_bytes = static_cast<const uint8_t*>(p.a);
    const uint8_t* const b_bytes = static_cast<const uint8_t*>(p.b);
    const int64_t row_bytes = static_cast<int64_t>(K) * ELEM;
    const int prow = lane >> 2, pch = lane & 3;

    const uint8_t* a_ptr[TS::LA];     // dense: row base + logical chunk offset
    int a_lchunk[TS::LA];             // logical chunk of this lane's slot
    bool a_rowok[TS::LA];
    int a_pix[!DENSE ? TS::LA : 1], a_h[!DENSE ? TS::LA : 1], a_w[!DENSE ? TS::LA : 1];
#pragma unroll
    for (int j = 0; j < TS::LA; ++j) {
        const int r = (wave * TS::LA + j) * kRowsPerLoad + prow;
        const int64_t m = m0 + r;
        a_rowok[j] = m < M;
        a_lchunk[j] = swz_chunk(r, pch);          // the swizzle is an involution
        if constexpr (DENSE) {
            a_ptr[j] = a_bytes + (a_rowok[j] ? m : 0) * row_bytes + a_lchunk[j] * 16;
        } else {
            const int mm = static_cast<int>(a_rowok[j] ? m : 0);
            const int hw = p.Ho * p.Wo;
            const int img = mm / hw, rem = mm - img * hw;
            const int ho = rem / p.Wo, wo = rem - ho * p.Wo;
            a_h[j] = ho * p.SH - p.PH;
            a_w[j] = wo * p.SW - p.PW;
            a_pix[j] = (img * p.H + a_h[j]) * p.W + a_w[j];
            a_ptr[j] = a_bytes;
        }
    }
    const uint8_t* b_ptr[TS::LB];
    int b_lchunk[TS::LB];
#pragma unroll
    for (int j = 0; j < TS::LB; ++j) {
        const int r = (wave * TS::LB + j) * kRowsPerLoad + prow;
        const int n = n0 + r;
        b_lchunk[j] = swz_chunk(r, pch);
        b_ptr[j] = (n < N) ? b_bytes + static_cast<int64_t>(n) * row_bytes + b_lchunk[j] * 16 : nullptr;
    }

    const void* const zp = g_zero_page;   // kept in registers across the loop
    // buffer form: this tile's A and B panels; rows past M or N lie outside and read zeros.
    // The host uses it only while 256 rows span less than 2 GB, so every offset fits.
    const int64_t a_rows = M - m0 < TS::BM ? M - m0 : TS::BM;
    const int b_rows = N - n0 < TS::BN ? N - n0 : TS::BN;
    const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(a_bytes + m0 * row_bytes, static_cast<uint32_t>(a_rows * row_bytes));
    const __amdgpu_buffer_rsrc_t b_rsrc =
        buffer_rsrc(b_bytes + static_cast<int64_t>(n0) * row_bytes, static_cast<uint32_t>(b_rows * row_bytes));
    uint32_t a_off[BUF ? TS::LA : 1], b_off[BUF ? TS::LB : 1];
    if constexpr (BUF) {
#pragma unroll
        for (int j = 0; j < TS::LA; ++j)
            a_off[j] = static_cast<uint32_t>(((wave * TS::LA + j) * kRowsPerLoad + prow) * row_bytes + a_lchunk[j] * 16);
#pragma unroll
        for (int j = 0; j < TS::LB; ++j)
            b_off[j] = static_cast<uint32_t>(((wave * TS::LB + j) * kRowsPerLoad + prow) * row_bytes + b_lchunk[j] * 16);
    }
    // Issues this lane's loads of slice kt (kt may exceed the last slice: then all zero
    // page).  sink(j, src, lds_dst) receives load slot j (A slots first, then B).
    auto gen_slice = [&](int kt, auto sink) {
        uint8_t* sA = smem + (kt % S) * TS::STAGE;
        uint8_t* sB = sA + TS::BM * kRowBytes;
        const int kbase = kt * KE;
        if constexpr (AMODE == kConvAligned) {
            // Cin % KE == 0: the whole slice lies in one kernel tap
            const bool kin = kbase < K;
            const int kb = kin ? kbase : 0;
            const int tap = kb / p.Cin;
            const int ci0 = kb - tap * p.Cin;
            const int r = tap / p.KW, s = tap - r * p.KW;
#pragma unroll
            for (int j = 0; j < TS::LA; ++j) {
                const int hi = a_h[j] + r, wi = a_w[j] + s;
                const bool ok = kin && a_rowok[j] && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                                static_cast<unsigned>(wi) < static_cast<unsigned>(p.W);
                const int64_t off =
                    (static_cast<int64_t>(a_pix[j] + r * p.W + s) * p.Cin + ci0 + a_lchunk[j] * CE) * ELEM;
                sink(j, ok ? static_cast<const void*>(a_bytes + off) : zp, sA + (wave * TS::LA + j) * 1024);
            }
        } else if constexpr (AMODE == kConvGeneric) {
#pragma unroll
            for (int j = 0; j < TS::LA; ++j) {
                const int k = kbase + a_lchunk[j] * CE;
                const bool kin = k < K;
                const int kc = kin ? k : 0;                     // division stays branch-free
                const int tap = kc / p.Cin, ci = kc - tap * p.Cin;
                const int r = tap / p.KW, s = tap - r * p.KW;
                const int hi = a_h[j] + r, wi = a_w[j] + s;
                const bool ok = kin && a_rowok[j] && static_cast<unsigned>(hi) < static_cast<unsigned>(p.H) &&
                                static_cast<unsigned>(wi) < static_cast<unsigned>(p.W);
                const int64_t off = (static_cast<int64_t>(a_pix[j] + r * p.W + s) * p.Cin + ci) * ELEM;
                sink(j, ok ? static_cast<const void*>(a_bytes + off) : zp, sA + (wave * TS::LA + j) * 1024);
            }
        } else if constexpr (AMODE == kConvAnyC) {
            // Any Cin: each of a chunk's 8 values is fetched on its own (zero outside the
            // image) and the chunk reaches LDS through registers, at the place the LDS-DMA
            // load would have put it.  Kernel row r covers the contiguous run t in [0, KW*Cin)
            // of input row a_h + r from column a_w on, so k = r*KW*Cin + t needs one division
            // per chunk and the column test is a range test on a_w*Cin + t.  The weight rows
            // (K values, K not a multiple of 8) are not 16-byte aligned either and are read
            // the same way, with zeros past K and past N.
            static_assert(ELEM == 2, "bf16 gather");
            const uint16_t* const xs = static_cast<const uint16_t*>(p.a);
            const int RK = p.KW * p.Cin, WC = p.W * p.Cin;
#pragma unroll
            for (int j = 0; j < TS::LA; ++j) {
                const int k0 = kbase + a_lchunk[j] * CE;
                int r = k0 / RK;
                int t = k0 - r * RK;
                const int q0 = a_w[j] * p.Cin;
                uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    const bool ok = a_rowok[j] && k0 + e < K &&
                                    static_cast<unsigned>(a_h[j] + r) < static_cast<unsigned>(p.H) &&
                                    static_cast<unsigned>(q0 + t) < static_cast<unsigned>(WC);
                    uint32_t val = 0u;
                    if (ok) val = xs[static_cast<int64_t>(a_pix[j] + r * p.W) * p.Cin + t];
                    v[e >> 1] |= val << (16 * (e & 1));
                    if (++t == RK) { t = 0; ++r; }
                }
                *reinterpret_cast<u32x4_t*>(sA + (wave * TS::LA + j) * 1024 + lane * 16) =
                    u32x4_t{v[0], v[1], v[2], v[3]};
            }
            const uint16_t* const ws = static_cast<const uint16_t*>(p.b);
#pragma unroll
            for (int j = 0; j < TS::LB; ++j) {
                const int n = n0 + (wave * TS::LB + j) * kRowsPerLoad + prow;
                const int k0 = kbase + b_lchunk[j] * CE;
                uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    uint32_t val = 0u;
                    if (n < N && k0 + e < K) val = ws[static_cast<int64_t>(n) * K + k0 + e];
                    v[e >> 1] |= val << (16 * (e & 1));
                }
                *reinterpret_cast<u32x4_t*>(sB + (wave * TS::LB + j) * 1024 + lane * 16) =
                    u32x4_t{v[0], v[1], v[2], v[3]};
            }
            return;
        } else if constexpr (BUF) {
#pragma unroll
            for (int j = 0; j < TS::LA; ++j) {
                const bool ok = kbase + a_lchunk[j] * CE < K;
                load_lds16_buf(a_rsrc, ok ? a_off[j] + static_cast<uint32_t>(kt * kRowBytes) : kOutOfRange,
                               sA + (wave * TS::LA + j) * 1024);
            }
#pragma unroll
            for (int j = 0; j < TS::LB; ++j) {
                const bool ok = kbase + b_lchunk[j] * CE < K;
                load_lds16_buf(b_rsrc, ok ? b_off[j] + static_cast<uint32_t>(kt * kRowBytes) : kOutOfRange,
                               sB + (wave * TS::LB + j) * 1024);
            }
            return;
        } else {
#pragma unroll
            for (int j = 0; j < TS::LA; ++j) {
                const bool ok = a_rowok[j] && kbase + a_lchunk[j] * CE < K;
                sink(j, ok ? static_cast<const void*>(a_ptr[j] + static_cast<int64_t>(kt) * kRowBytes) : zp,
                     sA + (wave * TS::LA + j) * 1024);
            }
        }
#pragma unroll
        for (int j = 0; j < TS::LB; ++j) {
            const bool ok = b_ptr[j] != nullptr && kbase + b_lchunk[j] * CE < K;
            sink(TS::LA + j, ok ? static_cast<const void*>(b_ptr[j] + static_cast<int64_t>(kt) * kRowBytes) : zp,
                 sB + (wave * TS::LB + j) * 1024);
        }
    };
    // LDS-DMA path: every load lands in LDS directly
    auto issue_slice = [&](int kt) {
        gen_slice(kt, [&](int, const void* src, uint8_t* dst) { load_lds16(src, dst); });
    };
    f32x16_t acc[TS::FN][TS::FM];     // D = W . X^T: acc[j][i] covers columns of fragment j, rows of i
#pragma unroll
    for (int j = 0; j < TS::FN; ++j)
#pragma unroll
        for (int i = 0; i < TS::FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // ---- software pipeline, branch-free.  Step g runs FM*FN MFMAs on the fragments in
    //      register buffer g&1 while the next step's fragments are read from LDS into the
    //      other buffer.  Every SPB slices there is a transition: this wave waits until its
    //      own loads of the next SPB slices have landed (later slices may stay in flight),
    //      then a barrier proves that every wave has them and that every wave is done
    //      reading the SPB slices just consumed, whose LDS buffers are refilled with the
    //      slices S ahead right away.  Slices past the end of K are read from the zero page,
    //      so every transition issues the same number of loads and the wait counts are
    //      constants; the K loop is padded with zero slices to a whole number of unrolled
    //      iterations for the same reason. ----
    constexpr int SPB = TS::SPB;
    typename F::T xf[2][TS::FM], wf[2][TS::FN];
    const int x_row = wm * TS::WTM + (lane & 31);   // activation fragment rows in the tile
    const int w_row = wn * TS::WTN + (lane & 31);   // weight fragment rows in the tile
    constexpr int P = SPB * F::kSteps;               // steps between transitions
    // steps per loop iteration: even (static fragment buffers)
    constexpr int U = P >= 2 ? P : 2;
    constexpr int SLICES_PER_ITER = U / F::kSteps;
    const int KTP = (KT + SLICES_PER_ITER - 1) / SLICES_PER_ITER * SLICES_PER_ITER;
    const int steps = KTP * F::kSteps;
    auto stage_a = [&](int kt) -> const uint8_t* { return smem + (kt % S) * TS::STAGE; };
    auto read_frags = [&](auto buf_c, int kt, int st) {
        constexpr int b = decltype(buf_c)::value;
        const uint8_t* sA = stage_a(kt);
#pragma unroll
        for (int i = 0; i < TS::FM; ++i) xf[b][i] = F::load(sA, x_row + 32 * i, st, lane);
#pragma unroll
        for (int j = 0; j < TS::FN; ++j) wf[b][j] = F::load(sA + TS::BM * kRowBytes, w_row + 32 * j, st, lane);
    };
    auto mma_all = [&](auto buf_c) {
        constexpr int b = decltype(buf_c)::value;
#pragma unroll
        for (int j = 0; j < TS::FN; ++j)
#pragma unroll
            for (int i = 0; i < TS::FM; ++i) acc[j][i] = F::mma(wf[b][j], xf[b][i], acc[j][i]);
    };
    constexpr int MF = TS::FM * TS::FN, R = (TS::FM + TS::FN) * F::kReads;
    auto schedule = [&](auto r_c, auto g_c, auto w_c) {
        interleave<MF, decltype(r_c)::value, decltype(g_c)::value, decltype(w_c)::value>();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) issue_slice(s2);
    wait_vmcnt<(S - SPB) * LOADS>();
    barrier();
    read_frags(I0{}, 0, 0);

    // step q of an unrolled iteration starting at step g0 (q and everything derived from it
    // are compile-time constants)
    auto step = [&](auto q_c, int g0) {
        constexpr int q = decltype(q_c)::value;
        constexpr int c = q & 1, n = c ^ 1;
        constexpr int st = q % F::kSteps;
        constexpr int slice_in_iter = q / F::kSteps;
        constexpr bool same_slice = st + 1 < F::kSteps;
        constexpr bool transition = !same_slice && (slice_in_iter + 1) % SPB == 0;
        const int kt = g0 / F::kSteps + slice_in_iter;
        if constexpr (same_slice) {
            read_frags(std::integral_constant<int, n>{}, kt, st + 1);
            mma_all(std::integral_constant<int, c>{});
            schedule(std::integral_constant<int, R>{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        } else if constexpr (!transition) {
            // the next slice landed at the previous transition
            read_frags(std::integral_constant<int, n>{}, kt + 1, 0);
            mma_all(std::integral_constant<int, c>{});
            schedule(std::integral_constant<int, R>{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        } else {
            wait_vmcnt<(S - 2 * SPB) * LOADS>();
            barrier();
#pragma unroll
            for (int i = 0; i < SPB; ++i) issue_slice(kt + 1 - SPB + S + i);
            read_frags(std::integral_constant<int, n>{}, kt + 1, 0);
            mma_all(std::integral_constant<int, c>{});
            schedule(std::integral_constant<int, R>{}, std::integral_constant<int, SPB * LOADS>{},
                     std::integral_constant<int, 0>{});
        }
    };
    for (int g = 0; g < steps; g += U) {
        step(std::integral_constant<int, 0>{}, g);
        step(std::integral_constant<int, 1>{}, g);
        if constexpr (U > 2) {
            step(std::integral_constant<int, 2>{}, g);
            step(std::integral_constant<int, 3>{}, g);
        }
    }

    mma_epilogue<TS, AMODE, ACT, OUT>(p, acc, smem, wm, wn, lane, tid, m0, n0);
}

// The tiles the library chooses from (api.cpp, pick_tile): the sixteen-wave 256 x 256 tile with
// one barrier per two K slices for large dense GEMMs (four waves per SIMD, each 64 x 64: 1 KB of
// LDS reads per MFMA, against 0.75 KB with eight waves of 128 x 64, but four waves to hide each
// other's read latency; 3.5-4.5% faster on the large GEMMs), and four-wave tiles for everything
// smaller and for the implicit-GEMM convolution.
using T256x256 = TileShape<256, 256, 4, 4, 4, 2>;
using T128x128 = TileShape<128, 128, 2, 2, 4>;
using T128x64 = TileShape<128, 64, 2, 2, 4>;
using T64x64 = TileShape<64, 64, 2, 2, 4>;

template <int ELEM, class TS, int AMODE, int ACT, int OUT>
hipError_t launch_one(const MmaArgs& a, hipStream_t stream) {
    const int64_t tm64 = (a.M + TS::BM - 1) / TS::BM;
    const int tiles_n = (a.N + TS::BN - 1) / TS::BN;
    if (tm64 * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>(tm64);
    if (tiles_m == 0 || tiles_n == 0) return hipSuccess;
    hipLaunchKernelGGL((mma_kernel<ELEM, TS, AMODE, ACT, OUT>), dim3(tiles_m * tiles_n), dim3(TS::NT), 0,
                       stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int ELEM, int AMODE, int ACT, int OUT>
hipError_t launch_tile(const MmaArgs& a, int tile, hipStream_t s) {
    switch (tile) {
        case kTile128x128: return launch_one<ELEM, T128x128, AMODE, ACT, OUT>(a, s);
        case kTile128x64: return launch_one<ELEM, T128x64, AMODE, ACT, OUT>(a, s);
        case kTile64x64: return launch_one<ELEM, T64x64, AMODE, ACT, OUT>(a, s);
        default: break;
    }
    if constexpr (AMODE == kDense || AMODE == kDenseWide) {
        if (tile == kTile256x256) return launch_one<ELEM, T256x256, AMODE, ACT, OUT>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace dlf
