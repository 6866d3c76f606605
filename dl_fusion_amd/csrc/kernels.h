// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlf {

// Route and tile switches (tuning and tests).  They are read from the environment once, when
// the library is loaded, and again by dlf_tuning_reload():
//   DLF_TILE=<n>            force MFMA tile n (a kTile* value the route has)
//   DLF_GEMM=tiled|stream   the tiled MFMA kernel, or the streaming kernel wherever it applies
//   DLF_CONV=generic|stream the implicit GEMM for every conv, or the weight-streaming halo kernel
//                           for every 3x3 stride-1 conv
//   DLF_STREAM_NB=128|256|384  the streaming kernel's column block, where built and dividing N
//   DLF_FFN_TOK=32|64       the fused FFN's token block
//   DLF_FFN_SPLIT=<s>       the fused FFN's d_ff parts (0 or 1: no split)
struct Options {
    int tile;        // forced tile, or -1
    int gemm;        // 0 the library's choice, 1 tiled only, 2 streaming where it applies
    int conv;        // 0 the library's choice, 1 implicit GEMM, 2 weight-streaming halo kernel
    int stream_nb;   // 0, or the forced column block
    int ffn_tok;     // 0, or the forced token block
    int ffn_split;   // 0 the library's choice, 1 no split, >= 2 that many parts
};
const Options& options();
void reload_options();

// Arguments of the MFMA GEMM / implicit-GEMM kernel.  C[m][n] = sum_k A[m][k] B[n][k]
// followed by the register epilogue.  For a convolution, A is gathered on the fly
// from the NHWC input (row m = (img, ho, wo), k = (r*KW + s)*Cin + ci).
struct MmaArgs {
    const void* a;          // dense: A [M][K]; conv: x [N][H][W][Cin]
    const void* b;          // B [N][K] (OHWI-flattened weights)
    const float* scale;     // [N] per-column multiplier or nullptr (= 1)
    const float* shift;     // [N] per-column bias / shift or nullptr (= 0)
    const uint16_t* res;    // bf16 residual [M][N] or nullptr
    void* c;                // output [M][N]
    int64_t M;
    int N, K;
    float out_inv_scale;    // fp8 output: fp32(1/s_y)
    float dequant;          // fp32 output of the plain fp8 GEMM: s_x * s_w
    // split store (parts > 1): columns [p * part_cols, (p + 1) * part_cols) go to outs[p], each
    // [M][part_cols]; part_cols is a multiple of one 16-byte chunk of output.  parts == 1: c.
    int parts, part_cols;
    void* outs[4];
    // convolution geometry (A gather); unused by the dense kernel
    int H, W, Cin, Ho, Wo, KW, SH, SW, PH, PW;
};

// Output tile shapes of the MFMA kernel (rows x columns of C per workgroup).  The 256 x 256
// tile serves the dense GEMM only; the implicit-GEMM convolution takes the other three.
enum MmaTile : int {
    kTile256x256 = 0,   // 4x4 waves of 64x64, one barrier per two K slices
    kTile128x128 = 1,   // 2x2 waves of 64x64
    kTile128x64 = 2,    // 2x2 waves of 64x32
    kTile64x64 = 3,     // 2x2 waves of 32x32
    kTileCount = 4
};
int mma_tile_rows(int tile);
int mma_tile_cols(int tile);

// out: kOutBf16 / kOutFp8 / kOutF32; act: kActNone / kActRelu / kActGelu.
hipError_t launch_mma_bf16(const MmaArgs& args, bool conv, int act, int tile, hipStream_t stream);
hipError_t launch_mma_fp8(const MmaArgs& args, int act, int out, int tile, hipStream_t stream);
// Streaming GEMM for memory-bound shapes (bf16, no scale, one output): K of 128 or 256, N a
// multiple of 128 (column blocks of 128 to 384, at most 32 of them), A and C below 2 GB.
bool gemm_stream_ok(const MmaArgs& args);
// ... and where it is faster than the tiled kernel (from 4M outputs)
bool gemm_stream_pays(const MmaArgs& args);
hipError_t launch_gemm_stream(const MmaArgs& args, int act, hipStream_t stream);
// instantiation groups of the MFMA kernel (one translation unit each); wide: rows of 8 MB or
// more, read by 64-bit global addresses
hipError_t launch_mma_bf16_dense(const MmaArgs& args, bool wide, int act, int tile, hipStream_t stream);
hipError_t launch_mma_bf16_gated(const MmaArgs& args, bool wide, int act, int tile, hipStream_t stream);
hipError_t launch_mma_bf16_conv(const MmaArgs& args, int act, int tile, hipStream_t stream);
hipError_t launch_mma_fp8_q(const MmaArgs& args, bool wide, int act, int tile, hipStream_t stream);
hipError_t launch_mma_fp8_b(const MmaArgs& args, bool wide, int act, int out, int tile, hipStream_t stream);

// fp32 direct convolution with the same epilogue (bias -> residual -> act).
struct ConvF32Args {
    const float* x;
    const float* w;
    const float* bias;      // nullable
    const float* res;       // nullable
    float* y;
    int M;                  // n * ho * wo (<= 2^30, checked on the host)
    int Cout, K;
    int H, W, Cin, Ho, Wo, KW, SH, SW, PH, PW;
};
hipError_t launch_conv_f32(const ConvF32Args& args, int act, hipStream_t stream);

// bf16 3x3 stride-1 pad-1 convolution with the input halo resident in LDS.
struct HaloArgs {
    const uint16_t* x;      // [N][H][W][Cin]
    const uint16_t* w;      // [Cout][3][3][Cin]
    const float* bias;      // [Cout] or nullptr
    const uint16_t* res;    // [N][H][W][Cout] or nullptr
    uint16_t* y;            // [N][H][W][Cout]
    int N, H, W, Cin, Cout;
    int co_tiles;           // Cout / 64
};
struct HaloPlan {
    int kind;        // 0: one row tile per workgroup, weights streamed; 1: Cin = 64, weights resident;
                     // 2: small images, one image x 32 output channels per workgroup
    int th;          // output rows per tile
    int row_tiles;   // ceil(H / th)
    int wf;          // 32-pixel fragments per wave (1 or 2)
    int halo_kb;     // LDS reserved for one halo
    int per_xcd;     // kind 1: spatial tiles per XCD
};
// False when the shape does not qualify (Cin = 64 or a multiple of 128, Cout a
// multiple of 64, the halo of one output row within 96 KB; or, for kind 2, Cin a
// multiple of 64, Cout of 32 and a small image).  resident_ok = false restricts the
// plan to the streaming kernel (kind 0).
bool conv_halo_plan(int N, int H, int W, int Cin, int Cout, bool resident_ok, HaloPlan* plan);
hipError_t launch_conv_halo(const HaloArgs& args, const HaloPlan& plan, int act, hipStream_t stream);

// bf16 convolution for inputs with few channels (c_in <= 4, e.g. a ResNet stem): weights and
// the input patch of `th` output rows re-laid in LDS with 4-channel pixels, one workgroup
// per CU with compute and store waves.
struct SmallCArgs {
    const uint16_t* x;      // [N][H][W][Cin]
    const uint16_t* w;      // [Cout][KH][KW][Cin]
    const float* bias;      // [Cout] or nullptr
    const uint16_t* res;    // [N][Ho][Wo][Cout] or nullptr
    uint16_t* y;            // [N][Ho][Wo][Cout]
    int N, H, W, Cin, Cout, KH, KW, SH, SW, PH, PW, Ho, Wo;
    int kwp;                // KW + toff rounded up to a multiple of 4
    int pw;                 // patch width in pixels (even)
    int pwl;                // patch column of image column 0: PW rounded up to even
    int toff;               // pwl - PW: kernel column s is tap s + toff
    int th;                 // output rows per workgroup
    int row_tiles;          // ceil(Ho / th)
    int co_blocks;          // ceil(Cout / 64)
};
// False when the shape does not qualify (Cin <= 4, Cout a multiple of 32, W*Cin a multiple
// of 8, KW + toff <= 16, and the weights of 64 channels, 64 KB of staged output and the
// patch of one output row within 160 KB of LDS); fills everything but the pointers.
bool conv_smallc_plan(int N, int H, int W, int Cin, int Cout, int KH, int KW, int SH, int SW, int PH, int PW,
                      int Ho, int Wo, SmallCArgs* args);
hipError_t launch_conv_smallc(const SmallCArgs& args, int act, hipStream_t stream);

// Feed-forward block FC1 -> act -> FC2 (+ b2, + residual) in one kernel; weights packed in
// MFMA fragment order (dlf_ffn_pack).
struct FfnArgs {
    const uint16_t* x;      // [M][D]
    const uint16_t* w1p;    // W1 [F][D], packed
    const float* b1;        // [F] or nullptr
    const uint16_t* w2p;    // W2 [D][F], packed
    const float* b2;        // [D] or nullptr
    const uint16_t* res;    // [M][D] or nullptr
    uint16_t* y;            // [M][D]
    int64_t M;
    int D, F;               // D in {256, 512, 768, 1024}; F a positive multiple of 256
    // parts S > 1: S workgroups a token block, each over 1/S of d_ff, write fp32 partial sums
    // of y to ws [S][M][D], which a second kernel adds with b2 and the residual
    int parts;
    float* ws;
};
// the d_ff parts the fused FFN splits into for these sizes (1 = no split); DLF_FFN_SPLIT=<S>
// forces S (0 or 1: no split) where a split is built
int ffn_parts(int64_t M, int D, int F);
hipError_t launch_ffn(const FfnArgs& args, int act, hipStream_t stream);

// Shader-clock probe: workgroups x 4 waves of back-to-back bf16 MFMAs; stamps[4 b + 0..3] =
// s_memtime before / after, s_memrealtime before / after, for workgroup b.
hipError_t launch_clock_probe(int workgroups, int iters, uint64_t* stamps, hipStream_t stream);

// Elementwise passes of the unfused chain.  dt: 0 fp32, 1 bf16.
hipError_t launch_bn_apply(int64_t rows, int64_t c, int dt, const void* y, const float* gamma,
                           const float* beta, const float* mean, const float* var, float eps,
                           void* z, hipStream_t stream);
hipError_t launch_scale_shift(int64_t rows, int64_t c, int dt, const void* y, const float* scale,
                              const float* shift, void* z, hipStream_t stream);
hipError_t launch_add(int64_t count, int dt, const void* a, const void* b, void* out,
                      hipStream_t stream);
hipError_t launch_act(int64_t count, int dt, int act, const void* in, void* out, hipStream_t stream);
hipError_t launch_quant(int64_t count, const float* in, float inv_scale, uint8_t* codes,
                        hipStream_t stream);

}  // namespace dlf
