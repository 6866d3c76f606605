// C ABI of libdlfusion: argument validation, host-side BN folding, kernel
// selection and launch.  Every check happens before the first HIP call, so a
// rejected call has no device-side effect.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/dlfusion.h"
#include "device_common.h"
#include "kernels.h"
#include "status.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace dlf {

dlf_status fail(dlf_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

dlf_status ok() {
    g_last_error[0] = '\0';
    return DLF_OK;
}

namespace {

Options read_options() {
    Options o{-1, 0, 0, 0, 0, 0};
    if (const char* e = std::getenv("DLF_TILE")) {
        const int t = std::atoi(e);
        if (t >= 0 && t < kTileCount) o.tile = t;
    }
    if (const char* e = std::getenv("DLF_GEMM")) o.gemm = std::strcmp(e, "tiled") == 0 ? 1 : std::strcmp(e, "stream") == 0 ? 2 : 0;
    if (const char* e = std::getenv("DLF_CONV")) o.conv = std::strcmp(e, "generic") == 0 ? 1 : std::strcmp(e, "stream") == 0 ? 2 : 0;
    if (const char* e = std::getenv("DLF_STREAM_NB")) {
        const int nb = std::atoi(e);
        if (nb == 128 || nb == 256 || nb == 384) o.stream_nb = nb;
    }
    if (const char* e = std::getenv("DLF_FFN_TOK")) {
        const int t = std::atoi(e);
        if (t == 32 || t == 64) o.ffn_tok = t;
    }
    if (const char* e = std::getenv("DLF_FFN_SPLIT")) {
        const int v = std::atoi(e);
        o.ffn_split = v <= 1 ? 1 : v;
    }
    return o;
}

// read once at library load (static initialisation), replaced only by dlf_tuning_reload
Options g_options = read_options();

}  // namespace

const Options& options() { return g_options; }
void reload_options() { g_options = read_options(); }

}  // namespace dlf

namespace {

using dlf::fail;
using dlf::ok;

dlf_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DLF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(dlf_dtype d) {
    switch (d) {
        case DLF_F32: return 4;
        case DLF_BF16: return 2;
        case DLF_FP8_E4M3: return 1;
    }
    return 0;
}

bool valid_dtype(int d) { return d == DLF_F32 || d == DLF_BF16 || d == DLF_FP8_E4M3; }
bool valid_act(int a) {
    return a == DLF_ACT_NONE || a == DLF_ACT_RELU || a == DLF_ACT_GELU_TANH || a == DLF_ACT_GELU_ERF;
}

// Byte ranges [p, p + n) overlap?
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Tile of the MFMA kernel for an M x N output.  A tile forced by DLF_TILE wins where the route
// has it (tuning only).  Otherwise the estimate is (rounds of 256 concurrent tiles) x (tile
// area / relative MFMA efficiency of the tile shape).  The 256 x 256 tile is the sixteen-wave
// pipeline with one barrier per two K slices (dense GEMMs only): its eight-wave predecessor
// was measured 7-10% faster than four waves of 128 x 128 on the 4096 x 11008 x 4096 bf16 and
// 8192 x 4096 x 4096 fp8 GEMMs, and sixteen waves another 3.5-4.5%.
// Memory-bound GEMMs (many rows, short K, narrow N) take the streaming kernel unless a tile
// is forced or DLF_GEMM=tiled asks for the tiled kernel; DLF_GEMM=stream takes it wherever it
// applies (tests of both routes).
bool stream_gemm(const dlf::MmaArgs& a) {
    const dlf::Options& o = dlf::options();
    if (o.tile >= 0 || o.gemm == 1) return false;
    if (o.gemm == 2) return dlf::gemm_stream_ok(a);
    return dlf::gemm_stream_pays(a);
}

int pick_tile(int64_t M, int64_t N, bool dense) {
    const int forced = dlf::options().tile;
    if (forced >= 0 && (dense || forced != dlf::kTile256x256)) return forced;
    // Measured on MI355X: four-wave 256x128 and 256x64 tiles lost to 128x128 / 128x64 on
    // every shape swept (memory-bound 1x1 layers, FFN projections, square GEMMs), and a
    // four-wave 256x256 tile of the implicit GEMM to 128x128.
    const int cands[] = {dlf::kTile256x256, dlf::kTile128x128, dlf::kTile128x64, dlf::kTile64x64};
    const double eff[] = {1.0, 0.8, 0.65, 0.5};
    int best = dlf::kTile64x64;
    double best_cost = 0;
    for (int i = dense ? 0 : 1; i < 4; ++i) {
        const int t = cands[i];
        const int64_t bm = dlf::mma_tile_rows(t), bn = dlf::mma_tile_cols(t);
        if (bn > 64 && N <= bn / 2) continue;   // mostly-empty columns
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        const int64_t rounds = (tiles + 255) / 256;
        const double cost = static_cast<double>(rounds) * static_cast<double>(bm * bn) / eff[i];
        if (best_cost == 0 || cost < best_cost) {
            best = t;
            best_cost = cost;
        }
    }
    return best;
}

int act_code(dlf_act a) {
    switch (a) {
        case DLF_ACT_RELU: return dlf::kActRelu;
        case DLF_ACT_GELU_TANH: return dlf::kActGelu;
        case DLF_ACT_GELU_ERF: return dlf::kActGeluErf;
        default: return dlf::kActNone;
    }
}

// Single round-to-nearest-even of a binary64 value to bfloat16 (no pass
// through binary32, so no double rounding).
uint16_t bf16_from_double(double v) {
    if (std::isnan(v)) return 0x7FC0;
    if (v == 0.0 || std::isinf(v)) {
        float f = static_cast<float>(v);
        uint32_t b;
        std::memcpy(&b, &f, 4);
        return static_cast<uint16_t>(b >> 16);
    }
    int e = 0;
    std::frexp(v, &e);                 // |v| in [2^(e-1), 2^e)
    int lead = e - 1;
    if (lead < -126) lead = -126;      // bf16 subnormals share the 2^-133 spacing
    const double ulp = std::ldexp(1.0, lead - 7);
    const double q = std::nearbyint(v / ulp) * ulp;   // exact scaling; RNE in the default mode
    const float f = static_cast<float>(q);             // exact, or +-inf on overflow
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return static_cast<uint16_t>(b >> 16);
}

struct ConvGeom {
    int64_t ho, wo, M, K;
};

dlf_status check_conv(const dlf_conv_desc* d, const void* x, const void* w, const float* bias,
                      const void* residual, const void* y, ConvGeom* g) {
    if (!d) return fail(DLF_ERR_INVALID_ARG, "conv descriptor is NULL");
    if (!valid_dtype(d->dtype)) return fail(DLF_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(d->dtype));
    if (!valid_act(d->act)) return fail(DLF_ERR_INVALID_ARG, "unknown activation %d", static_cast<int>(d->act));
    if (d->n < 0 || d->h < 0 || d->w < 0 || d->c_in < 0 || d->c_out < 0)
        return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (d->kh <= 0 || d->kw <= 0) return fail(DLF_ERR_INVALID_ARG, "kernel extent must be positive");
    if (d->stride_h <= 0 || d->stride_w <= 0) return fail(DLF_ERR_INVALID_ARG, "stride must be positive");
    if (d->pad_h < 0 || d->pad_w < 0) return fail(DLF_ERR_INVALID_ARG, "padding must be non-negative");
    const int64_t hp = d->h + 2 * static_cast<int64_t>(d->pad_h), wp = d->w + 2 * static_cast<int64_t>(d->pad_w);
    g->ho = hp >= d->kh ? (hp - d->kh) / d->stride_h + 1 : 0;
    g->wo = wp >= d->kw ? (wp - d->kw) / d->stride_w + 1 : 0;
    g->M = d->n * g->ho * g->wo;
    g->K = d->kh * d->kw * d->c_in;
    if (d->dtype == DLF_FP8_E4M3) return fail(DLF_ERR_UNSUPPORTED, "fp8 convolution has no fused kernel");
    // 32-bit index limits of the kernels (the value-by-value gather for c_in % 8 != 0 also
    // indexes a whole image row, w * c_in, in 32 bits)
    const int64_t lim = int64_t(1) << 30;
    if (d->n * d->h * d->w > lim || g->K > lim || d->c_out > lim || d->h > lim || d->w > lim ||
        g->ho * g->wo > lim || d->n * (d->h + d->kh) * (d->w + d->kw) > lim || d->w * d->c_in > lim)
        return fail(DLF_ERR_UNSUPPORTED, "tensor too large for 32-bit pixel indexing");
    if (g->M == 0 || d->c_out == 0) return ok();
    if (!y || (g->K > 0 && (!x || !w)))
        return fail(DLF_ERR_INVALID_ARG, "x, w and y must be non-NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)) ||
        (residual && !aligned16(residual)))
        return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t es = dtype_size(d->dtype);
    const size_t ybytes = static_cast<size_t>(g->M * d->c_out) * es;
    if (overlaps(y, ybytes, x, static_cast<size_t>(d->n * d->h * d->w * d->c_in) * es) ||
        overlaps(y, ybytes, w, static_cast<size_t>(d->c_out * g->K) * es) ||
        overlaps(y, ybytes, bias, static_cast<size_t>(d->c_out) * 4) ||
        overlaps(y, ybytes, residual, ybytes))
        return fail(DLF_ERR_ALIAS, "output overlaps an input");
    return ok();
}

dlf_status launch_conv(const dlf_conv_desc* d, const ConvGeom& g, const void* x, const void* w,
                       const float* bias, const void* residual, void* y, void* stream, const char* what) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d->dtype == DLF_F32) {
        dlf::ConvF32Args a{};
        a.x = static_cast<const float*>(x);
        a.w = static_cast<const float*>(w);
        a.bias = bias;
        a.res = static_cast<const float*>(residual);
        a.y = static_cast<float*>(y);
        a.M = static_cast<int>(g.M);
        a.Cout = static_cast<int>(d->c_out);
        a.K = static_cast<int>(g.K);
        a.H = static_cast<int>(d->h); a.W = static_cast<int>(d->w); a.Cin = static_cast<int>(d->c_in);
        a.Ho = static_cast<int>(g.ho); a.Wo = static_cast<int>(g.wo); a.KW = static_cast<int>(d->kw);
        a.SH = d->stride_h; a.SW = d->stride_w; a.PH = d->pad_h; a.PW = d->pad_w;
        return hip_status(dlf::launch_conv_f32(a, act_code(d->act), s), what);
    }
    // 3x3, stride 1, pad 1: the halo kernels; at most four input channels: the small-channel
    // kernel.  DLF_CONV=generic forces the implicit GEMM, DLF_CONV=stream the halo kernel
    // that streams weights (tests of every route).
    dlf::HaloPlan plan{};
    const bool generic = dlf::options().conv == 1;
    const bool stream_only = dlf::options().conv == 2;
    dlf::SmallCArgs sc{};
    if (!generic && g.K > 0 &&
        dlf::conv_smallc_plan(static_cast<int>(d->n), static_cast<int>(d->h), static_cast<int>(d->w),
                              static_cast<int>(d->c_in), static_cast<int>(d->c_out), static_cast<int>(d->kh),
                              static_cast<int>(d->kw), d->stride_h, d->stride_w, d->pad_h, d->pad_w,
                              static_cast<int>(g.ho), static_cast<int>(g.wo), &sc)) {
        sc.x = static_cast<const uint16_t*>(x);
        sc.w = static_cast<const uint16_t*>(w);
        sc.bias = bias;
        sc.res = static_cast<const uint16_t*>(residual);
        sc.y = static_cast<uint16_t*>(y);
        return hip_status(dlf::launch_conv_smallc(sc, act_code(d->act), s), what);
    }
    if (!generic && g.K > 0 && d->kh == 3 && d->kw == 3 && d->stride_h == 1 && d->stride_w == 1 &&
        d->pad_h == 1 && d->pad_w == 1 &&
        dlf::conv_halo_plan(static_cast<int>(d->n), static_cast<int>(d->h), static_cast<int>(d->w),
                            static_cast<int>(d->c_in), static_cast<int>(d->c_out), !stream_only, &plan)) {
        dlf::HaloArgs h{};
        h.x = static_cast<const uint16_t*>(x);
        h.w = static_cast<const uint16_t*>(w);
        h.bias = bias;
        h.res = static_cast<const uint16_t*>(residual);
        h.y = static_cast<uint16_t*>(y);
        h.N = static_cast<int>(d->n); h.H = static_cast<int>(d->h); h.W = static_cast<int>(d->w);
        h.Cin = static_cast<int>(d->c_in); h.Cout = static_cast<int>(d->c_out);
        h.co_tiles = h.Cout / 64;
        return hip_status(dlf::launch_conv_halo(h, plan, act_code(d->act), s), what);
    }
    dlf::MmaArgs a{};
    a.a = x;
    a.b = w;
    a.scale = nullptr;
    a.shift = bias;
    a.res = static_cast<const uint16_t*>(residual);
    a.c = y;
    a.M = g.M;
    a.N = static_cast<int>(d->c_out);
    a.K = static_cast<int>(g.K);
    a.out_inv_scale = 1.0f;
    a.dequant = 1.0f;
    // a 1x1, stride-1, unpadded conv is the GEMM of the [n*h*w][c_in] pixel matrix: the dense
    // kernel reads it with buffer loads and no gather arithmetic
    if (!generic && d->kh == 1 && d->kw == 1 && d->stride_h == 1 && d->stride_w == 1 && d->pad_h == 0 &&
        d->pad_w == 0 && d->c_in % 8 == 0) {
        if (stream_gemm(a)) return hip_status(dlf::launch_gemm_stream(a, act_code(d->act), s), what);
        return hip_status(dlf::launch_mma_bf16(a, false, act_code(d->act), pick_tile(g.M, d->c_out, true), s), what);
    }
    a.H = static_cast<int>(d->h); a.W = static_cast<int>(d->w); a.Cin = static_cast<int>(d->c_in);
    a.Ho = static_cast<int>(g.ho); a.Wo = static_cast<int>(g.wo); a.KW = static_cast<int>(d->kw);
    a.SH = d->stride_h; a.SW = d->stride_w; a.PH = d->pad_h; a.PW = d->pad_w;
    // a strided, unpadded 1x1 conv (a ResNet downsample) reads every SH-th row and SW-th pixel:
    // the streaming kernel gathers those rows into its ring
    if (!generic && d->kh == 1 && d->kw == 1 && d->pad_h == 0 && d->pad_w == 0 && stream_gemm(a))
        return hip_status(dlf::launch_gemm_stream(a, act_code(d->act), s), what);
    // the value-by-value gather (c_in % 8 != 0) is latency-bound: smaller tiles, more of them
    const int tile = d->c_in % 8 != 0 && dlf::options().tile < 0 ? static_cast<int>(dlf::kTile128x64)
                                                                 : pick_tile(g.M, d->c_out, false);
    return hip_status(dlf::launch_mma_bf16(a, true, act_code(d->act), tile, s), what);
}

dlf_status check_gemm_common(const dlf_gemm_desc* d, const void* a, const void* b, const void* c) {
    if (!d) return fail(DLF_ERR_INVALID_ARG, "gemm descriptor is NULL");
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype))
        return fail(DLF_ERR_INVALID_ARG, "unknown dtype");
    if (!valid_act(d->act)) return fail(DLF_ERR_INVALID_ARG, "unknown activation %d", static_cast<int>(d->act));
    if (d->m < 0 || d->n < 0 || d->k < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (d->n > (int64_t(1) << 30) || d->k > (int64_t(1) << 30))
        return fail(DLF_ERR_UNSUPPORTED, "n and k must stay below 2^30");
    if (d->in_dtype == DLF_BF16 && d->k % 8 != 0)
        return fail(DLF_ERR_UNSUPPORTED, "bf16 GEMM needs k %% 8 == 0");
    if (d->in_dtype == DLF_FP8_E4M3 && d->k % 16 != 0)
        return fail(DLF_ERR_UNSUPPORTED, "fp8 GEMM needs k %% 16 == 0");
    if (d->m == 0 || d->n == 0) return ok();
    if (!c || (d->k > 0 && (!a || !b))) return fail(DLF_ERR_INVALID_ARG, "a, b and c must be non-NULL");
    if (!aligned16(a) || !aligned16(b) || !aligned16(c))
        return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    return ok();
}

}  // namespace

extern "C" {

const char* dlf_status_string(dlf_status s) {
    switch (s) {
        case DLF_OK: return "DLF_OK";
        case DLF_ERR_INVALID_ARG: return "DLF_ERR_INVALID_ARG";
        case DLF_ERR_UNSUPPORTED: return "DLF_ERR_UNSUPPORTED";
        case DLF_ERR_HIP: return "DLF_ERR_HIP";
        case DLF_ERR_ALIAS: return "DLF_ERR_ALIAS";
    }
    return "DLF_STATUS_UNKNOWN";
}

const char* dlf_last_error(void) { return g_last_error; }

void dlf_tuning_reload(void) { dlf::reload_options(); }

dlf_status dlf_clock_probe(int32_t workgroups, int32_t iters, uint64_t* stamps, void* stream) {
    if (workgroups < 1 || workgroups > 65536 || iters < 1)
        return fail(DLF_ERR_INVALID_ARG, "workgroups must be in [1, 65536] and iters >= 1");
    if (!stamps || !aligned16(stamps)) return fail(DLF_ERR_INVALID_ARG, "stamps must be a 16-byte aligned device pointer");
    return hip_status(dlf::launch_clock_probe(workgroups, iters, stamps, static_cast<hipStream_t>(stream)),
                      "dlf_clock_probe");
}

dlf_status dlf_fold_bn(int64_t cout, int64_t k, const float* w, const float* conv_bias, const float* gamma,
                       const float* beta, const float* mean, const float* var, double eps,
                       dlf_dtype w_out_dtype, void* w_out, float* bias_out) {
    if (cout < 0 || k < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (!std::isfinite(eps) || eps < 0.0) return fail(DLF_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (w_out_dtype != DLF_F32 && w_out_dtype != DLF_BF16) {
        if (!valid_dtype(w_out_dtype)) return fail(DLF_ERR_INVALID_ARG, "unknown dtype");
        return fail(DLF_ERR_UNSUPPORTED, "folded weights are produced in fp32 or bf16 only");
    }
    if (cout == 0) return ok();
    if (!gamma || !beta || !mean || !var || !bias_out || (k > 0 && (!w || !w_out)))
        return fail(DLF_ERR_INVALID_ARG, "NULL pointer argument");
    for (int64_t c = 0; c < cout; ++c) {
        const double den = static_cast<double>(var[c]) + eps;
        if (!(den > 0.0) || !std::isfinite(den))
            return fail(DLF_ERR_INVALID_ARG, "var + eps must be > 0 (channel %lld)", static_cast<long long>(c));
    }
    for (int64_t c = 0; c < cout; ++c) {
        const double s = static_cast<double>(gamma[c]) / std::sqrt(static_cast<double>(var[c]) + eps);
        const double b = conv_bias ? static_cast<double>(conv_bias[c]) : 0.0;
        bias_out[c] = static_cast<float>((b - static_cast<double>(mean[c])) * s + static_cast<double>(beta[c]));
        const float* wr = w + c * k;
        if (w_out_dtype == DLF_F32) {
            float* o = static_cast<float*>(w_out) + c * k;
            for (int64_t j = 0; j < k; ++j) o[j] = static_cast<float>(static_cast<double>(wr[j]) * s);
        } else {
            uint16_t* o = static_cast<uint16_t*>(w_out) + c * k;
            for (int64_t j = 0; j < k; ++j) o[j] = bf16_from_double(static_cast<double>(wr[j]) * s);
        }
    }
    return ok();
}

dlf_status dlf_bn_scale_shift(int64_t cout, const float* conv_bias, const float* gamma, const float* beta,
                              const float* mean, const float* var, double eps, double pre_scale,
                              float* scale_out, float* shift_out) {
    if (cout < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (!std::isfinite(eps) || eps < 0.0) return fail(DLF_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!std::isfinite(pre_scale)) return fail(DLF_ERR_INVALID_ARG, "pre_scale must be finite");
    if (cout == 0) return ok();
    if (!gamma || !beta || !mean || !var || !scale_out || !shift_out)
        return fail(DLF_ERR_INVALID_ARG, "NULL pointer argument");
    for (int64_t c = 0; c < cout; ++c) {
        const double den = static_cast<double>(var[c]) + eps;
        if (!(den > 0.0) || !std::isfinite(den))
            return fail(DLF_ERR_INVALID_ARG, "var + eps must be > 0 (channel %lld)", static_cast<long long>(c));
    }
    for (int64_t c = 0; c < cout; ++c) {
        const double s = static_cast<double>(gamma[c]) / std::sqrt(static_cast<double>(var[c]) + eps);
        const double b = conv_bias ? static_cast<double>(conv_bias[c]) : 0.0;
        scale_out[c] = static_cast<float>(pre_scale * s);
        shift_out[c] = static_cast<float>((b - static_cast<double>(mean[c])) * s + static_cast<double>(beta[c]));
    }
    return ok();
}

dlf_status dlf_conv_fused(const dlf_conv_desc* d, const void* x, const void* w, const float* bias,
                          const void* residual, void* y, void* stream) {
    ConvGeom g;
    const dlf_status st = check_conv(d, x, w, bias, residual, y, &g);
    if (st != DLF_OK || g.M == 0 || d->c_out == 0) return st;
    return launch_conv(d, g, x, w, bias, residual, y, stream, "dlf_conv_fused");
}

dlf_status dlf_conv_plain(const dlf_conv_desc* d, const void* x, const void* w, const float* conv_bias, void* y,
                          void* stream) {
    ConvGeom g;
    const dlf_status st = check_conv(d, x, w, conv_bias, nullptr, y, &g);
    if (st != DLF_OK) return st;
    if (d->act != DLF_ACT_NONE) return fail(DLF_ERR_INVALID_ARG, "the plain convolution applies no activation");
    if (g.M == 0 || d->c_out == 0) return ok();
    return launch_conv(d, g, x, w, conv_bias, nullptr, y, stream, "dlf_conv_plain");
}

}  // extern "C"

namespace {

// dlf_gemm_fused and its split-store form: parts == 0 stores c as [m][n]; parts >= 1 stores
// columns [p n/parts, (p+1) n/parts) to outs[p].
dlf_status gemm_fused_impl(const dlf_gemm_desc* d, const void* a, const void* b, const float* col_scale,
                           const float* col_shift, const void* residual, void* c, int parts, void* const* outs,
                           void* stream, const char* what) {
    void* const first = parts > 0 ? (outs ? outs[0] : nullptr) : c;
    dlf_status st = check_gemm_common(d, a, b, first);
    if (st != DLF_OK) return st;
    const bool bf16_path = d->in_dtype == DLF_BF16 && d->out_dtype == DLF_BF16;
    const bool fp8_path = d->in_dtype == DLF_FP8_E4M3 &&
                          (d->out_dtype == DLF_FP8_E4M3 || d->out_dtype == DLF_BF16) &&
                          residual == nullptr;
    if (!bf16_path && !fp8_path)
        return fail(DLF_ERR_UNSUPPORTED, "no fused GEMM for in=%d out=%d act=%d residual=%s",
                    static_cast<int>(d->in_dtype), static_cast<int>(d->out_dtype), static_cast<int>(d->act),
                    residual ? "yes" : "no");
    if (d->out_dtype == DLF_FP8_E4M3 && (!std::isfinite(d->out_inv_scale) || !(d->out_inv_scale > 0.0f)))
        return fail(DLF_ERR_INVALID_ARG, "out_inv_scale must be finite and > 0");
    const size_t in_es = dtype_size(d->in_dtype), out_es = dtype_size(d->out_dtype);
    int part_cols = 0;
    if (parts > 0) {
        if (parts > 4) return fail(DLF_ERR_UNSUPPORTED, "at most 4 output parts");
        if (residual) return fail(DLF_ERR_UNSUPPORTED, "the split store takes no residual");
        if (d->n % parts != 0) return fail(DLF_ERR_INVALID_ARG, "n must split into %d equal parts", parts);
        part_cols = static_cast<int>(d->n / parts);
        if ((static_cast<size_t>(part_cols) * out_es) % 16 != 0)
            return fail(DLF_ERR_UNSUPPORTED, "each part's row must be a whole number of 16-byte chunks");
    }
    if (d->m == 0 || d->n == 0) return ok();
    if ((col_scale && !aligned16(col_scale)) || (col_shift && !aligned16(col_shift)) ||
        (residual && !aligned16(residual)))
        return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t abytes = static_cast<size_t>(d->m * d->k) * in_es, bbytes = static_cast<size_t>(d->n * d->k) * in_es;
    auto clobbers_input = [&](const void* out, size_t bytes) {
        return overlaps(out, bytes, a, abytes) || overlaps(out, bytes, b, bbytes) ||
               overlaps(out, bytes, col_scale, static_cast<size_t>(d->n) * 4) ||
               overlaps(out, bytes, col_shift, static_cast<size_t>(d->n) * 4) || overlaps(out, bytes, residual, bytes);
    };
    dlf::MmaArgs x{};
    if (parts > 0) {
        const size_t pbytes = static_cast<size_t>(d->m) * part_cols * out_es;
        for (int q = 0; q < parts; ++q) {
            if (!outs[q] || !aligned16(outs[q]))
                return fail(DLF_ERR_INVALID_ARG, "output part %d is NULL or not 16-byte aligned", q);
            if (clobbers_input(outs[q], pbytes)) return fail(DLF_ERR_ALIAS, "output part %d overlaps an input", q);
            for (int r = 0; r < q; ++r)
                if (overlaps(outs[q], pbytes, outs[r], pbytes))
                    return fail(DLF_ERR_ALIAS, "output parts %d and %d overlap", r, q);
            x.outs[q] = outs[q];
        }
        x.parts = parts;
        x.part_cols = part_cols;
        x.c = outs[0];
    } else {
        if (clobbers_input(c, static_cast<size_t>(d->m * d->n) * out_es))
            return fail(DLF_ERR_ALIAS, "output overlaps an input");
        x.c = c;
    }
    x.a = a;
    x.b = b;
    x.scale = col_scale;
    x.shift = col_shift;
    x.res = static_cast<const uint16_t*>(residual);
    x.M = d->m;
    x.N = static_cast<int>(d->n);
    x.K = static_cast<int>(d->k);
    x.out_inv_scale = d->out_inv_scale;
    x.dequant = 1.0f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bf16_path && stream_gemm(x)) return hip_status(dlf::launch_gemm_stream(x, act_code(d->act), s), what);
    const int tile = pick_tile(d->m, d->n, true);
    if (bf16_path) return hip_status(dlf::launch_mma_bf16(x, false, act_code(d->act), tile, s), what);
    const int out = d->out_dtype == DLF_FP8_E4M3 ? dlf::kOutFp8 : dlf::kOutBf16;
    return hip_status(dlf::launch_mma_fp8(x, act_code(d->act), out, tile, s), what);
}

}  // namespace

extern "C" {

dlf_status dlf_gemm_fused(const dlf_gemm_desc* d, const void* a, const void* b, const float* col_scale,
                          const float* col_shift, const void* residual, void* c, void* stream) {
    return gemm_fused_impl(d, a, b, col_scale, col_shift, residual, c, 0, nullptr, stream, "dlf_gemm_fused");
}

dlf_status dlf_gemm_fused_gated(const dlf_gemm_desc* d, const void* a, const void* b, const float* col_scale,
                                const float* col_shift, dlf_gate gate, void* c, void* stream) {
    if (!d) return fail(DLF_ERR_INVALID_ARG, "gemm descriptor is NULL");
    if (gate != DLF_GATE_SILU && gate != DLF_GATE_GELU_TANH && gate != DLF_GATE_GELU_ERF)
        return fail(DLF_ERR_INVALID_ARG, "unknown gate %d", static_cast<int>(gate));
    if (d->act != DLF_ACT_NONE) return fail(DLF_ERR_INVALID_ARG, "the gate replaces the activation: act must be NONE");
    const dlf_status st = check_gemm_common(d, a, b, c);
    if (st != DLF_OK) return st;
    if (d->in_dtype != DLF_BF16 || d->out_dtype != DLF_BF16)
        return fail(DLF_ERR_UNSUPPORTED, "gated epilogue: bf16 operands and output only");
    if (d->n % 2 != 0) return fail(DLF_ERR_INVALID_ARG, "n must be even: (gate, up) column pairs");
    if (d->m == 0 || d->n == 0) return ok();
    if ((col_scale && !aligned16(col_scale)) || (col_shift && !aligned16(col_shift)))
        return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t cbytes = static_cast<size_t>(d->m) * static_cast<size_t>(d->n / 2) * 2;
    if (overlaps(c, cbytes, a, static_cast<size_t>(d->m * d->k) * 2) ||
        overlaps(c, cbytes, b, static_cast<size_t>(d->n * d->k) * 2) ||
        overlaps(c, cbytes, col_scale, static_cast<size_t>(d->n) * 4) ||
        overlaps(c, cbytes, col_shift, static_cast<size_t>(d->n) * 4))
        return fail(DLF_ERR_ALIAS, "output overlaps an input");
    dlf::MmaArgs x{};
    x.a = a;
    x.b = b;
    x.scale = col_scale;
    x.shift = col_shift;
    x.c = c;
    x.M = d->m;
    x.N = static_cast<int>(d->n);
    x.K = static_cast<int>(d->k);
    x.out_inv_scale = 1.0f;
    x.dequant = 1.0f;
    const int act = gate == DLF_GATE_SILU ? dlf::kActSiluMul : gate == DLF_GATE_GELU_TANH ? dlf::kActGeluMul
                                                                                           : dlf::kActGeluErfMul;
    return hip_status(dlf::launch_mma_bf16(x, false, act, pick_tile(d->m, d->n, true), static_cast<hipStream_t>(stream)),
                      "dlf_gemm_fused_gated");
}

dlf_status dlf_gemm_fused_split(const dlf_gemm_desc* d, const void* a, const void* b, const float* col_scale,
                                const float* col_shift, int32_t parts, void* const* outs, void* stream) {
    if (parts < 1) return fail(DLF_ERR_INVALID_ARG, "parts must be >= 1");
    if (!outs) return fail(DLF_ERR_INVALID_ARG, "outs is NULL");
    return gemm_fused_impl(d, a, b, col_scale, col_shift, nullptr, nullptr, parts, outs, stream,
                           "dlf_gemm_fused_split");
}

dlf_status dlf_gemm_plain(const dlf_gemm_desc* d, const void* a, const void* b, float dequant, void* y,
                          void* stream) {
    dlf_status st = check_gemm_common(d, a, b, y);
    if (st != DLF_OK) return st;
    if (d->act != DLF_ACT_NONE) return fail(DLF_ERR_INVALID_ARG, "the plain GEMM applies no activation");
    const bool bf16_path = d->in_dtype == DLF_BF16 && d->out_dtype == DLF_BF16;
    const bool fp8_path = d->in_dtype == DLF_FP8_E4M3 && d->out_dtype == DLF_F32;
    if (!bf16_path && !fp8_path) return fail(DLF_ERR_UNSUPPORTED, "no plain GEMM for this dtype pair");
    if (fp8_path && !std::isfinite(dequant)) return fail(DLF_ERR_INVALID_ARG, "dequant must be finite");
    if (d->m == 0 || d->n == 0) return ok();
    const size_t in_es = dtype_size(d->in_dtype), out_es = dtype_size(d->out_dtype);
    const size_t ybytes = static_cast<size_t>(d->m * d->n) * out_es;
    if (overlaps(y, ybytes, a, static_cast<size_t>(d->m * d->k) * in_es) ||
        overlaps(y, ybytes, b, static_cast<size_t>(d->n * d->k) * in_es))
        return fail(DLF_ERR_ALIAS, "output overlaps an input");
    dlf::MmaArgs x{};
    x.a = a;
    x.b = b;
    x.c = y;
    x.M = d->m;
    x.N = static_cast<int>(d->n);
    x.K = static_cast<int>(d->k);
    x.out_inv_scale = 1.0f;
    x.dequant = dequant;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int tile = pick_tile(d->m, d->n, true);
    if (bf16_path) return hip_status(dlf::launch_mma_bf16(x, false, dlf::kActNone, tile, s), "dlf_gemm_plain");
    return hip_status(dlf::launch_mma_fp8(x, dlf::kActNone, dlf::kOutF32, tile, s), "dlf_gemm_plain");
}

static dlf_status check_eltwise(int64_t count, dlf_dtype dt, const void* in, const void* out) {
    if (count < 0) return fail(DLF_ERR_INVALID_ARG, "negative size");
    if (!valid_dtype(dt)) return fail(DLF_ERR_INVALID_ARG, "unknown dtype");
    if (dt == DLF_FP8_E4M3) return fail(DLF_ERR_UNSUPPORTED, "elementwise passes take fp32 or bf16");
    if (count == 0) return ok();
    if (!in || !out) return fail(DLF_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned16(in) || !aligned16(out)) return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    return ok();
}

dlf_status dlf_bn_apply(int64_t rows, int64_t c, dlf_dtype dt, const void* y, const float* gamma,
                        const float* beta, const float* mean, const float* var, double eps, void* z,
                        void* stream) {
    if (rows < 0 || c < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    if (!std::isfinite(eps) || eps < 0.0) return fail(DLF_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const int64_t count = rows * c;
    dlf_status st = check_eltwise(count, dt, y, z);
    if (st != DLF_OK || count == 0) return st;
    if (!gamma || !beta || !mean || !var) return fail(DLF_ERR_INVALID_ARG, "NULL BN parameter");
    const size_t bytes = static_cast<size_t>(count) * dtype_size(dt);
    if (overlaps(z, bytes, y, bytes) && z != y) return fail(DLF_ERR_ALIAS, "output partially overlaps the input");
    return hip_status(dlf::launch_bn_apply(rows, c, dt == DLF_F32 ? 0 : 1, y, gamma, beta, mean, var,
                                           static_cast<float>(eps), z, static_cast<hipStream_t>(stream)),
                      "dlf_bn_apply");
}

dlf_status dlf_scale_shift_apply(int64_t rows, int64_t c, dlf_dtype dt, const void* y, const float* scale,
                                 const float* shift, void* z, void* stream) {
    if (rows < 0 || c < 0) return fail(DLF_ERR_INVALID_ARG, "negative dimension");
    const int64_t count = rows * c;
    dlf_status st = check_eltwise(count, dt, y, z);
    if (st != DLF_OK || count == 0) return st;
    if (!shift) return fail(DLF_ERR_INVALID_ARG, "shift must be non-NULL");
    const size_t bytes = static_cast<size_t>(count) * dtype_size(dt);
    if (overlaps(z, bytes, y, bytes) && z != y) return fail(DLF_ERR_ALIAS, "output partially overlaps the input");
    return hip_status(dlf::launch_scale_shift(rows, c, dt == DLF_F32 ? 0 : 1, y, scale, shift, z,
                                              static_cast<hipStream_t>(stream)),
                      "dlf_scale_shift_apply");
}

dlf_status dlf_add(int64_t count, dlf_dtype dt, const void* a, const void* b, void* out, void* stream) {
    dlf_status st = check_eltwise(count, dt, a, out);
    if (st != DLF_OK || count == 0) return st;
    if (!b) return fail(DLF_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned16(b)) return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    const size_t bytes = static_cast<size_t>(count) * dtype_size(dt);
    if ((overlaps(out, bytes, a, bytes) && out != a) || (overlaps(out, bytes, b, bytes) && out != b))
        return fail(DLF_ERR_ALIAS, "output partially overlaps an input");
    return hip_status(dlf::launch_add(count, dt == DLF_F32 ? 0 : 1, a, b, out, static_cast<hipStream_t>(stream)),
                      "dlf_add");
}

dlf_status dlf_act_apply(int64_t count, dlf_dtype dt, dlf_act act, const void* in, void* out, void* stream) {
    if (!valid_act(act)) return fail(DLF_ERR_INVALID_ARG, "unknown activation %d", static_cast<int>(act));
    dlf_status st = check_eltwise(count, dt, in, out);
    if (st != DLF_OK || count == 0) return st;
    const size_t bytes = static_cast<size_t>(count) * dtype_size(dt);
    if (overlaps(out, bytes, in, bytes) && out != in) return fail(DLF_ERR_ALIAS, "output partially overlaps the input");
    return hip_status(dlf::launch_act(count, dt == DLF_F32 ? 0 : 1, act_code(act), in, out,
                                      static_cast<hipStream_t>(stream)),
                      "dlf_act_apply");
}

dlf_status dlf_quant_apply(int64_t count, const float* in, float inv_scale, uint8_t* codes, void* stream) {
    if (count < 0) return fail(DLF_ERR_INVALID_ARG, "negative size");
    if (!std::isfinite(inv_scale) || !(inv_scale > 0.0f)) return fail(DLF_ERR_INVALID_ARG, "inv_scale must be finite and > 0");
    if (count == 0) return ok();
    if (!in || !codes) return fail(DLF_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned16(in) || !aligned16(codes)) return fail(DLF_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (overlaps(codes, static_cast<size_t>(count), in, static_cast<size_t>(count) * 4))
        return fail(DLF_ERR_ALIAS, "output overlaps the input");
    return hip_status(dlf::launch_quant(count, in, inv_scale, codes, static_cast<hipStream_t>(stream)),
                      "dlf_quant_apply");
}

}  // extern "C"
